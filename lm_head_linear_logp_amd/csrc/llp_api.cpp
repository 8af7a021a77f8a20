// llp_api.cpp -- the C-ABI entry points: request validation, workspace layout and the launch
// sequences of the fused linear log-prob operator. Validation is plain C++ that runs before
// any HIP call, so a malformed request is rejected without touching a device.
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "llp.h"
#include "llp_internal.h"

using namespace llp;

namespace {

thread_local char g_err[512] = "";

llp_status fail(llp_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

#define LLP_CHECK(cond, st, ...) \
  do {                           \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

constexpr int kMaxDevices = 64;
std::mutex g_mu;
int g_opened[kMaxDevices] = {0};
int g_num_cus[kMaxDevices] = {0};

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

int64_t local_real(const llp_vocab_partition& v) {
  int64_t n = v.real_vocab - v.offset;
  if (n < 0) n = 0;
  if (n > v.local_size) n = v.local_size;
  return n;
}

llp_status check_partition(const llp_vocab_partition& v) {
  LLP_CHECK(v.world >= 1 && v.world <= LLP_MAX_WORLD, LLP_ERR_INVALID_ARGUMENT,
            "vocab.world=%d outside [1, %d]", v.world, LLP_MAX_WORLD);
  LLP_CHECK(v.rank >= 0 && v.rank < v.world, LLP_ERR_INVALID_ARGUMENT,
            "vocab.rank=%d outside [0, world=%d)", v.rank, v.world);
  LLP_CHECK(v.real_vocab > 0 && v.real_vocab <= v.padded_vocab, LLP_ERR_INVALID_ARGUMENT,
            "need 0 < real_vocab (%lld) <= padded_vocab (%lld)", (long long)v.real_vocab,
            (long long)v.padded_vocab);
  // Compared without forming offset + local_size, which could overflow.
  LLP_CHECK(v.offset >= 0 && v.local_size >= 0 && v.offset <= v.padded_vocab &&
                v.local_size <= v.padded_vocab - v.offset,
            LLP_ERR_INVALID_ARGUMENT, "shard [offset=%lld, +local_size=%lld) outside padded vocab %lld",
            (long long)v.offset, (long long)v.local_size, (long long)v.padded_vocab);
  if (v.world == 1)
    LLP_CHECK(v.offset == 0 && v.local_size == v.padded_vocab, LLP_ERR_INVALID_ARGUMENT,
              "world == 1 needs offset 0 and local_size == padded_vocab");
  LLP_CHECK(v.padded_vocab < (int64_t(1) << 31), LLP_ERR_UNSUPPORTED,
            "padded_vocab %lld exceeds int32 indexing", (long long)v.padded_vocab);
  return LLP_OK;
}

llp_status check_request(const llp_request* req) {
  LLP_CHECK(req != nullptr, LLP_ERR_INVALID_ARGUMENT, "request is NULL");
  const llp_projection& p = req->proj;
  const int64_t T = req->layout.num_tokens;
  LLP_CHECK(T >= 0, LLP_ERR_INVALID_ARGUMENT, "num_tokens=%lld < 0", (long long)T);
  LLP_CHECK(T <= (int64_t(1) << 23) - 256, LLP_ERR_UNSUPPORTED, "num_tokens %lld too large",
            (long long)T);
  llp_status st = check_partition(req->vocab);
  if (st != LLP_OK) return st;
  LLP_CHECK(p.hidden_size > 0, LLP_ERR_INVALID_ARGUMENT, "hidden_size must be > 0");
  LLP_CHECK(p.hidden_size % 64 == 0 && p.hidden_size <= (1 << 20), LLP_ERR_UNSUPPORTED,
            "hidden_size %lld must be a multiple of 64 (and <= 2^20)", (long long)p.hidden_size);
  LLP_CHECK(p.hidden_stride >= p.hidden_size && p.hidden_stride % 8 == 0,
            LLP_ERR_INVALID_ARGUMENT, "hidden_stride %lld must be >= H and a multiple of 8",
            (long long)p.hidden_stride);
  LLP_CHECK(p.weight_stride >= p.hidden_size && p.weight_stride % 8 == 0,
            LLP_ERR_INVALID_ARGUMENT, "weight_stride %lld must be >= H and a multiple of 8",
            (long long)p.weight_stride);
  // Operand rows are addressed with 32-bit byte offsets from a tile's first row.
  LLP_CHECK(p.hidden_stride < (int64_t(1) << 23) && p.weight_stride < (int64_t(1) << 23),
            LLP_ERR_UNSUPPORTED, "hidden_stride and weight_stride must be < 2^23");
  // The fused tiles gather hidden rows through one buffer resource per tile, based at the
  // tile's first scored row, with 32-bit byte offsets: every byte of the T rows must lie below
  // 2^31 from the base.
  LLP_CHECK(T * p.hidden_stride * 2 < (int64_t(1) << 31), LLP_ERR_UNSUPPORTED,
            "hidden spans T * hidden_stride * 2 = %lld bytes; must be < 2^31",
            (long long)(T * p.hidden_stride * 2));
  LLP_CHECK(req->vocab.local_size <= (int64_t(1) << 23) - 256, LLP_ERR_UNSUPPORTED,
            "local_size %lld exceeds 2^23 - 256", (long long)req->vocab.local_size);
  if (T > 0) {
    LLP_CHECK(p.hidden != nullptr, LLP_ERR_INVALID_ARGUMENT, "proj.hidden is NULL");
    LLP_CHECK(aligned(p.hidden, 16), LLP_ERR_INVALID_ARGUMENT, "proj.hidden not 16-byte aligned");
    LLP_CHECK(req->target_ids != nullptr, LLP_ERR_INVALID_ARGUMENT, "target_ids is NULL");
  }
  if (local_real(req->vocab) > 0) {
    LLP_CHECK(p.weight != nullptr, LLP_ERR_INVALID_ARGUMENT, "proj.weight is NULL");
    LLP_CHECK(aligned(p.weight, 16), LLP_ERR_INVALID_ARGUMENT, "proj.weight not 16-byte aligned");
  }
  if (p.bias != nullptr) {
    LLP_CHECK(p.bias_dtype == LLP_DTYPE_BF16 || p.bias_dtype == LLP_DTYPE_F32,
              LLP_ERR_INVALID_ARGUMENT, "bias_dtype %d is not BF16 or F32", p.bias_dtype);
    LLP_CHECK(aligned(p.bias, p.bias_dtype == LLP_DTYPE_F32 ? 16 : 8), LLP_ERR_INVALID_ARGUMENT,
              "proj.bias not %d-byte aligned", p.bias_dtype == LLP_DTYPE_F32 ? 16 : 8);
  }
  LLP_CHECK(isfinite(req->temperature) && req->temperature > 0.f, LLP_ERR_INVALID_ARGUMENT,
            "temperature must be finite and > 0");
  LLP_CHECK((req->flags & ~uint32_t(LLP_FLAG_WANT_ENTROPY | LLP_FLAG_OVERWRITE_GRADS |
                                    LLP_FLAG_G_SLABS)) == 0,
            LLP_ERR_INVALID_ARGUMENT, "unknown flags 0x%x", req->flags);
  if (req->layout.cu_seqlens != nullptr)
    LLP_CHECK(req->layout.num_seqs >= 0, LLP_ERR_INVALID_ARGUMENT, "num_seqs < 0");
  return LLP_OK;
}

// Workspace regions (byte offsets, each 256-byte aligned).
struct Ws {
  size_t count, qctr, scored, pos, tloc, tz, pm, ps, pq, G, hgT, P, dbp, total;
  int64_t T_cap, nvt, ldg;
  int64_t slab_tiles, nslab;   // vocabulary tiles per slab of G and slabs per backward call
};

// `slabs` (backward only): G is held one vocabulary slab of G_SLAB_TILES tiles at a time, so
// its region (and the bias-gradient partials) take one slab's columns, ldg = the slab width.
Ws ws_layout(int64_t T, int64_t n_real, int64_t H, int op, bool slabs = false) {
  Ws w{};
  w.T_cap = round_up(T > 0 ? T : 1, TILE);
  w.nvt = (n_real + TILE - 1) / TILE;
  w.slab_tiles = slabs && w.nvt > G_SLAB_TILES ? G_SLAB_TILES : (w.nvt > 0 ? w.nvt : 1);
  w.nslab = w.nvt > 0 ? (w.nvt + w.slab_tiles - 1) / w.slab_tiles : 0;
  w.ldg = w.slab_tiles * TILE;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (size_t)round_up((int64_t)(bytes > 0 ? bytes : 1), 256);
    return o;
  };
  w.count = take((size_t)(1 + layout_blocks(T)) * 4);   // 256 bytes up to 63 layout blocks
  // Tile-queue counters: QCTR_INTS per GEMM kernel launch of the call (3 per slab backward).
  w.qctr = take((size_t)(w.nslab > 1 ? 3 * w.nslab : 4) * QCTR_INTS * 4);
  w.scored = take((size_t)w.T_cap * 4);
  w.pos = take((size_t)w.T_cap * 4);
  w.tloc = take((size_t)w.T_cap * 4);
  if (op == LLP_OP_FORWARD) {
    w.tz = take((size_t)w.T_cap * 4);
    w.pm = take((size_t)(w.nvt * w.T_cap) * 4);
    w.ps = take((size_t)(w.nvt * w.T_cap) * 4);
    w.pq = take((size_t)(w.nvt * w.T_cap) * 4);
  } else {
    w.G = take((size_t)w.T_cap * (size_t)w.ldg * 2);    // G[j][v]
    w.hgT = take((size_t)H * (size_t)w.T_cap * 2);      // scored hidden rows, transposed
    w.P = take((size_t)DH_SPLITS * (size_t)w.T_cap * (size_t)H * 4);
    w.dbp = take((size_t)(w.T_cap / TILE) * (size_t)w.ldg * 4);   // bias-gradient partials
  }
  w.total = off;
  return w;
}

// The current device must have been opened; `num_cus` (optional) receives its compute units.
llp_status check_device(int* num_cus = nullptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(LLP_ERR_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_mu);
  LLP_CHECK(dev >= 0 && dev < kMaxDevices && g_opened[dev], LLP_ERR_INVALID_ARGUMENT,
            "llp_open has not succeeded on the current device %d", dev);
  if (num_cus) *num_cus = g_num_cus[dev];
  return LLP_OK;
}

llp_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return LLP_OK;
  return fail(LLP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define LLP_HIP(expr, what)                         \
  do {                                              \
    llp_status s_ = hip_status((expr), (what));     \
    if (s_ != LLP_OK) return s_;                    \
  } while (0)

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

}  // namespace

extern "C" {

// Rows of a logits view are read with 16-byte loads.
static bool rows_aligned(const void* p, int64_t stride, int64_t esize) {
  return p == nullptr || (aligned(p, 16) && (stride * esize) % 16 == 0);
}

LLP_API llp_status llp_forward_logits(const llp_logits_request* req, const llp_partials* out,
                                      void* stream) {
  LLP_CHECK(req != nullptr && out != nullptr, LLP_ERR_INVALID_ARGUMENT, "req/out is NULL");
  llp_status st = check_partition(req->vocab);
  if (st != LLP_OK) return st;
  const int64_t T = req->layout.num_tokens;
  LLP_CHECK(T >= 0 && T < (int64_t(1) << 31), LLP_ERR_INVALID_ARGUMENT, "num_tokens out of range");
  LLP_CHECK(req->logits_dtype == LLP_DTYPE_F32 || req->logits_dtype == LLP_DTYPE_BF16,
            LLP_ERR_INVALID_ARGUMENT, "logits_dtype %d is not F32 or BF16", req->logits_dtype);
  const int64_t esize = req->logits_dtype == LLP_DTYPE_F32 ? 4 : 2;
  LLP_CHECK(req->logits_stride >= req->vocab.local_size, LLP_ERR_INVALID_ARGUMENT,
            "logits_stride < local_size");
  LLP_CHECK(rows_aligned(req->logits, req->logits_stride, esize), LLP_ERR_INVALID_ARGUMENT,
            "logits rows must be 16-byte aligned (base and stride * element size)");
  LLP_CHECK(isfinite(req->temperature) && req->temperature > 0.f, LLP_ERR_INVALID_ARGUMENT,
            "temperature must be finite and > 0");
  LLP_CHECK((req->flags & ~uint32_t(LLP_FLAG_WANT_ENTROPY)) == 0, LLP_ERR_INVALID_ARGUMENT,
            "unknown flags 0x%x", req->flags);
  if (req->layout.cu_seqlens != nullptr)
    LLP_CHECK(req->layout.num_seqs >= 0, LLP_ERR_INVALID_ARGUMENT, "num_seqs < 0");
  if (T > 0) {
    LLP_CHECK(req->target_ids != nullptr, LLP_ERR_INVALID_ARGUMENT, "target_ids is NULL");
    LLP_CHECK(req->logits || local_real(req->vocab) == 0, LLP_ERR_INVALID_ARGUMENT,
              "logits is NULL");
    LLP_CHECK(out->target_logit && out->in_range && out->lse, LLP_ERR_INVALID_ARGUMENT,
              "out.target_logit, out.in_range and out.lse are required");
    LLP_CHECK(((req->flags & LLP_FLAG_WANT_ENTROPY) != 0) == (out->entropy != nullptr),
              LLP_ERR_INVALID_ARGUMENT, "out.entropy must be given exactly when entropy is wanted");
  }
  st = check_device();
  if (st != LLP_OK) return st;
  if (T == 0) return LLP_OK;
  LogitsArgs la{};
  la.T = T;
  la.logits = req->logits;
  la.bf16 = req->logits_dtype == LLP_DTYPE_BF16;
  la.ld = req->logits_stride;
  la.offset = req->vocab.offset;
  la.n_real = local_real(req->vocab);
  la.real_vocab = req->vocab.real_vocab;
  la.world = req->vocab.world;
  la.mask = req->layout.loss_mask;
  la.cu_seqlens = req->layout.cu_seqlens;
  la.num_seqs = req->layout.num_seqs;
  la.targets = req->target_ids;
  la.c1 = (float)(1.0 / (double)req->temperature);
  la.out_t = out->target_logit;
  la.out_f = out->in_range;
  la.out_l = out->lse;
  la.out_e = out->entropy;
  la.out_p = out->logp;
  la.status = req->status_word;
  LLP_HIP(launch_logits(la, static_cast<hipStream_t>(stream)), "logits forward kernel launch");
  return LLP_OK;
}

LLP_API llp_status llp_keep_mask_replay(const llp_keep_mask_request* req,
                                        const llp_partials* out, void* stream) {
  LLP_CHECK(req != nullptr && out != nullptr, LLP_ERR_INVALID_ARGUMENT, "req/out is NULL");
  llp_status st = check_partition(req->vocab);
  if (st != LLP_OK) return st;
  const int64_t T = req->num_tokens;
  LLP_CHECK(T >= 0 && T < (int64_t(1) << 31), LLP_ERR_INVALID_ARGUMENT, "num_tokens out of range");
  LLP_CHECK(req->processed_logprobs == 1, LLP_ERR_INVALID_ARGUMENT,
            "replay scores processed logprobs only (processed_logprobs must be 1)");
  LLP_CHECK(req->logits_dtype == LLP_DTYPE_F32 || req->logits_dtype == LLP_DTYPE_BF16,
            LLP_ERR_INVALID_ARGUMENT, "logits_dtype %d is not F32 or BF16", req->logits_dtype);
  const int64_t esize = req->logits_dtype == LLP_DTYPE_F32 ? 4 : 2;
  LLP_CHECK(req->logits_stride >= req->vocab.local_size, LLP_ERR_INVALID_ARGUMENT,
            "logits_stride < local_size");
  LLP_CHECK(rows_aligned(req->logits, req->logits_stride, esize), LLP_ERR_INVALID_ARGUMENT,
            "logits rows must be 16-byte aligned (base and stride * element size)");
  LLP_CHECK(req->keep_stride >= req->vocab.local_size, LLP_ERR_INVALID_ARGUMENT,
            "keep_stride < local_size");
  LLP_CHECK(rows_aligned(req->keep_mask, req->keep_stride, 1), LLP_ERR_INVALID_ARGUMENT,
            "keep_mask rows must be 16-byte aligned (base and stride)");
  LLP_CHECK(isfinite(req->temperature) && req->temperature > 0.f, LLP_ERR_INVALID_ARGUMENT,
            "temperature must be finite and > 0");
  LLP_CHECK(out->entropy == nullptr, LLP_ERR_INVALID_ARGUMENT,
            "replay produces no entropy (out.entropy must be NULL)");
  if (T > 0) {
    LLP_CHECK(req->target_ids != nullptr, LLP_ERR_INVALID_ARGUMENT, "target_ids is NULL");
    LLP_CHECK((req->logits && req->keep_mask) || local_real(req->vocab) == 0,
              LLP_ERR_INVALID_ARGUMENT, "logits and keep_mask are required");
    LLP_CHECK(out->target_logit && out->in_range && out->lse, LLP_ERR_INVALID_ARGUMENT,
              "out.target_logit, out.in_range and out.lse are required");
  }
  st = check_device();
  if (st != LLP_OK) return st;
  if (T == 0) return LLP_OK;
  KeepArgs ka{};
  ka.T = T;
  ka.logits = req->logits;
  ka.bf16 = req->logits_dtype == LLP_DTYPE_BF16;
  ka.lstride = req->logits_stride;
  ka.keep = req->keep_mask;
  ka.kstride = req->keep_stride;
  ka.offset = req->vocab.offset;
  ka.n_real = local_real(req->vocab);
  ka.real_vocab = req->vocab.real_vocab;
  ka.mask = req->loss_mask;
  ka.targets = req->target_ids;
  ka.c1 = (float)(1.0 / (double)req->temperature);
  ka.out_t = out->target_logit;
  ka.out_f = out->in_range;
  ka.out_l = out->lse;
  ka.out_p = out->logp;
  ka.status = req->status_word;
  LLP_HIP(launch_keep(ka, static_cast<hipStream_t>(stream)), "keep-mask replay kernel launch");
  return LLP_OK;
}

LLP_API const char* llp_last_error(void) { return g_err; }

LLP_API llp_status llp_open(int32_t device, llp_info* info) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0)
    return fail(LLP_ERR_UNAVAILABLE, "no HIP device is available");
  LLP_CHECK(device >= 0 && device < n && device < kMaxDevices, LLP_ERR_INVALID_ARGUMENT,
            "device %d outside [0, %d)", device, n);
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess)
    return fail(LLP_ERR_UNAVAILABLE, "hipGetDeviceProperties failed for device %d", device);
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(LLP_ERR_UNAVAILABLE, "device %d is %s; the kernels are built for gfx950", device,
                prop.gcnArchName);
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return fail(LLP_ERR_UNAVAILABLE, "hipGetDevice failed");
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (hipSetDevice(device) != hipSuccess)
      return fail(LLP_ERR_UNAVAILABLE, "hipSetDevice(%d) failed", device);
    const hipError_t pe = probe_kernels();
    // With the device current: its copy of the static scratch of llp_forward_noalloc.
    const hipError_t se = pe == hipSuccess ? scratch_init(device) : pe;
    (void)hipSetDevice(cur);
    if (pe != hipSuccess)
      return fail(LLP_ERR_UNAVAILABLE, "kernels cannot be loaded on device %d: %s", device,
                  hipGetErrorString(pe));
    if (se != hipSuccess)
      return fail(LLP_ERR_UNAVAILABLE, "static scratch not addressable on device %d: %s", device,
                  hipGetErrorString(se));
    g_opened[device] = 1;
    g_num_cus[device] = prop.multiProcessorCount;
  }
  if (info) {
    memset(info, 0, sizeof(*info));
    snprintf(info->name, sizeof(info->name), "lm_head_linear_logp_amd");
    snprintf(info->version, sizeof(info->version), "%s", LLP_VERSION);
    snprintf(info->arch, sizeof(info->arch), "%.31s", prop.gcnArchName);
    snprintf(info->route, sizeof(info->route),
             "hip-gfx950 mfma32x32x16bf16 tile256x256 bk64 lds-dma-2stage fwd-w8-persistent bwd-w4 xcd8 vgroup8 dhsplit%d",
             DH_SPLITS);
    info->max_replay_ids = LLP_MAX_REPLAY_IDS;
    info->num_cus = prop.multiProcessorCount;
    info->device = device;
  }
  return LLP_OK;
}

LLP_API llp_status llp_workspace_bytes(const llp_request* req, int32_t op, size_t* bytes) {
  llp_status st = check_request(req);
  if (st != LLP_OK) return st;
  LLP_CHECK(op == LLP_OP_FORWARD || op == LLP_OP_BACKWARD, LLP_ERR_INVALID_ARGUMENT,
            "op %d is not LLP_OP_FORWARD or LLP_OP_BACKWARD", op);
  LLP_CHECK(bytes != nullptr, LLP_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = ws_layout(req->layout.num_tokens, local_real(req->vocab), req->proj.hidden_size, op,
                     op == LLP_OP_BACKWARD && (req->flags & LLP_FLAG_G_SLABS) != 0).total;
  return LLP_OK;
}

}  // extern "C"

namespace {

// The forward of one shard on a caller's workspace (llp_forward) or the static scratch
// (llp_forward_noalloc): validation, then layout, fused tiles and combine on `stream`.
llp_status forward_impl(const llp_request* req, const llp_partials* out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  llp_status st = check_request(req);
  if (st != LLP_OK) return st;
  LLP_CHECK(out != nullptr, LLP_ERR_INVALID_ARGUMENT, "out is NULL");
  const int64_t T = req->layout.num_tokens;
  const bool want_ent = (req->flags & LLP_FLAG_WANT_ENTROPY) != 0;
  if (T > 0) {
    LLP_CHECK(out->target_logit && out->in_range && out->lse, LLP_ERR_INVALID_ARGUMENT,
              "out.target_logit, out.in_range and out.lse are required");
  }
  LLP_CHECK(T == 0 || !want_ent || out->entropy != nullptr, LLP_ERR_INVALID_ARGUMENT,
            "LLP_FLAG_WANT_ENTROPY needs out.entropy");
  const int64_t n_real = local_real(req->vocab);
  const int64_t H = req->proj.hidden_size;
  const Ws w = ws_layout(T, n_real, H, LLP_OP_FORWARD);
  LLP_CHECK(workspace_bytes >= w.total, LLP_ERR_INVALID_ARGUMENT,
            "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, w.total);
  LLP_CHECK(workspace != nullptr && aligned(workspace, 256), LLP_ERR_INVALID_ARGUMENT,
            "workspace must be non-NULL and 256-byte aligned");
  int num_cus = 0;
  st = check_device(&num_cus);
  if (st != LLP_OK) return st;
  if (T == 0) return LLP_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* ent = want_ent ? out->entropy : nullptr;

  LayoutArgs la{};
  la.T = T;
  la.mask = req->layout.loss_mask;
  la.cu_seqlens = req->layout.cu_seqlens;
  la.num_seqs = req->layout.num_seqs;
  la.world = req->vocab.world;
  la.targets = req->target_ids;
  la.offset = req->vocab.offset;
  la.n_real = n_real;
  la.real_vocab = req->vocab.real_vocab;
  la.count = at<int32_t>(workspace, w.count);
  la.scored = at<int32_t>(workspace, w.scored);
  la.pos = at<int32_t>(workspace, w.pos);
  la.tloc = at<int32_t>(workspace, w.tloc);
  la.out_t = out->target_logit;
  la.out_f = out->in_range;
  la.out_l = out->lse;
  la.out_e = ent;
  la.out_p = out->logp;
  la.status = req->status_word;
  la.qctr = at<int32_t>(workspace, w.qctr);   // the forward kernel's tile-queue counters
  la.nqctr = QCTR_INTS;
  LLP_HIP(launch_layout(la, s), "layout kernel launch");

  FwdArgs fa{};
  fa.W = static_cast<const uint16_t*>(req->proj.weight);
  fa.ldw = req->proj.weight_stride;
  fa.h = static_cast<const uint16_t*>(req->proj.hidden);
  fa.ldh = req->proj.hidden_stride;
  fa.bias = req->proj.bias;
  fa.bias_f32 = req->proj.bias_dtype == LLP_DTYPE_F32;
  fa.H = (int32_t)H;
  fa.n_real = n_real;
  fa.nvt = (int32_t)w.nvt;
  fa.ntb = (int32_t)(w.T_cap / TILE);
  fa.c1 = (float)(1.0 / (double)req->temperature);
  fa.count = la.count;
  fa.scored = la.scored;
  fa.tloc = la.tloc;
  fa.pm = at<float>(workspace, w.pm);
  fa.ps = at<float>(workspace, w.ps);
  fa.pq = at<float>(workspace, w.pq);
  fa.tz = at<float>(workspace, w.tz);
  fa.pstride = w.T_cap;
  fa.qctr = la.qctr;
  fa.workers = num_cus;
  LLP_HIP(launch_fwd(fa, s), "forward kernel launch");

  CombineArgs ca{};
  ca.nvt = (int32_t)w.nvt;
  ca.pstride = w.T_cap;
  ca.count = la.count;
  ca.scored = la.scored;
  ca.tloc = la.tloc;
  ca.pm = fa.pm;
  ca.ps = fa.ps;
  ca.pq = fa.pq;
  ca.tz = fa.tz;
  ca.out_t = out->target_logit;
  ca.out_f = out->in_range;
  ca.out_l = out->lse;
  ca.out_e = ent;
  ca.out_p = out->logp;
  LLP_HIP(launch_combine(ca, w.T_cap, s), "combine kernel launch");
  return LLP_OK;
}

}  // namespace

extern "C" {

LLP_API llp_status llp_forward(const llp_request* req, const llp_partials* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return forward_impl(req, out, workspace, workspace_bytes, stream);
}

LLP_API llp_status llp_forward_noalloc(const llp_request* req, const llp_partials* out,
                                       void* stream) {
  llp_status st = check_request(req);
  if (st != LLP_OK) return st;
  const size_t need = ws_layout(req->layout.num_tokens, local_real(req->vocab),
                                req->proj.hidden_size, LLP_OP_FORWARD).total;
  LLP_CHECK(need <= SCRATCH_BYTES, LLP_ERR_UNSUPPORTED,
            "the request needs %zu bytes of forward workspace; the static scratch holds %zu "
            "(use llp_forward with a caller workspace, or fewer rows per call)", need,
            SCRATCH_BYTES);
  st = check_device();
  if (st != LLP_OK) return st;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(LLP_ERR_HIP, "hipGetDevice failed");
  void* ws = scratch_address(dev);
  LLP_CHECK(ws != nullptr, LLP_ERR_INTERNAL, "static scratch not set up on device %d", dev);
  return forward_impl(req, out, ws, SCRATCH_BYTES, stream);
}

LLP_API llp_status llp_merge(int32_t world, const llp_partials* parts, int64_t num_tokens,
                             const uint8_t* loss_mask, const llp_final_out* out,
                             int32_t* status_word, void* stream) {
  LLP_CHECK(world >= 1 && world <= LLP_MAX_WORLD, LLP_ERR_INVALID_ARGUMENT,
            "world=%d outside [1, %d]", world, LLP_MAX_WORLD);
  LLP_CHECK(parts != nullptr && out != nullptr, LLP_ERR_INVALID_ARGUMENT, "parts/out is NULL");
  LLP_CHECK(num_tokens >= 0 && num_tokens < (int64_t(1) << 31), LLP_ERR_INVALID_ARGUMENT,
            "num_tokens=%lld out of range", (long long)num_tokens);
  const bool want_ent = out->entropy != nullptr;
  if (num_tokens > 0) {
    LLP_CHECK(out->logp && out->lse, LLP_ERR_INVALID_ARGUMENT, "out.logp and out.lse are required");
    for (int r = 0; r < world; ++r) {
      LLP_CHECK(parts[r].target_logit && parts[r].in_range && parts[r].lse,
                LLP_ERR_INVALID_ARGUMENT, "parts[%d] lacks target_logit/in_range/lse", r);
      LLP_CHECK(!want_ent || parts[r].entropy, LLP_ERR_INVALID_ARGUMENT,
                "out.entropy requested but parts[%d].entropy is NULL", r);
    }
  }
  llp_status st = check_device();
  if (st != LLP_OK) return st;
  if (num_tokens == 0) return LLP_OK;
  MergeArgs ma{};
  ma.T = num_tokens;
  ma.world = world;
  ma.mask = loss_mask;
  for (int r = 0; r < world; ++r) {
    ma.tl[r] = parts[r].target_logit;
    ma.flag[r] = parts[r].in_range;
    ma.lse[r] = parts[r].lse;
    ma.ent[r] = parts[r].entropy;
  }
  ma.out_p = out->logp;
  ma.out_l = out->lse;
  ma.out_e = out->entropy;
  ma.status = status_word;
  LLP_HIP(launch_merge(ma, static_cast<hipStream_t>(stream)), "merge kernel launch");
  return LLP_OK;
}

LLP_API llp_status llp_backward(const llp_request* req, const llp_bwd_in* in,
                                const llp_bwd_out* out, void* workspace, size_t workspace_bytes,
                                void* stream) {
  llp_status st = check_request(req);
  if (st != LLP_OK) return st;
  LLP_CHECK(in != nullptr && out != nullptr, LLP_ERR_INVALID_ARGUMENT, "in/out is NULL");
  const int64_t T = req->layout.num_tokens;
  const int64_t H = req->proj.hidden_size;
  const int64_t n_real = local_real(req->vocab);
  if (T > 0) {
    LLP_CHECK(in->lse && in->dlogp, LLP_ERR_INVALID_ARGUMENT, "in.lse and in.dlogp are required");
    LLP_CHECK(!in->dentropy || in->entropy, LLP_ERR_INVALID_ARGUMENT,
              "in.dentropy needs in.entropy");
    LLP_CHECK(out->dhidden != nullptr && aligned(out->dhidden, 16), LLP_ERR_INVALID_ARGUMENT,
              "out.dhidden must be non-NULL and 16-byte aligned");
    LLP_CHECK(out->dhidden_stride >= H && out->dhidden_stride % 8 == 0, LLP_ERR_INVALID_ARGUMENT,
              "dhidden_stride must be >= H and a multiple of 8");
  }
  if (req->vocab.local_size > 0) {
    LLP_CHECK(out->dweight != nullptr, LLP_ERR_INVALID_ARGUMENT, "out.dweight is NULL");
    LLP_CHECK(out->dweight_stride >= H, LLP_ERR_INVALID_ARGUMENT, "dweight_stride must be >= H");
    LLP_CHECK(out->dweight_stride % 4 == 0 && aligned(out->dweight, 16), LLP_ERR_INVALID_ARGUMENT,
              "dweight needs a 16-byte aligned base and a stride that is a multiple of 4");
    LLP_CHECK(out->dweight_stride < (int64_t(1) << 21), LLP_ERR_UNSUPPORTED,
              "dweight_stride must be < 2^21");
  }
  const Ws w = ws_layout(T, n_real, H, LLP_OP_BACKWARD, (req->flags & LLP_FLAG_G_SLABS) != 0);
  LLP_CHECK(workspace_bytes >= w.total, LLP_ERR_INVALID_ARGUMENT,
            "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, w.total);
  LLP_CHECK(workspace != nullptr && aligned(workspace, 256), LLP_ERR_INVALID_ARGUMENT,
            "workspace must be non-NULL and 256-byte aligned");
  st = check_device();
  if (st != LLP_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool overwrite = (req->flags & LLP_FLAG_OVERWRITE_GRADS) != 0;
  // Overwrite mode: rows the products do not write (padding rows; every row when the call has
  // no rows) are written as 0.
  if (overwrite) {
    ZeroArgs za{};
    za.p = out->dweight;
    za.ld = out->dweight_stride;
    za.r0 = T == 0 ? 0 : n_real;
    za.r1 = req->vocab.local_size;
    za.cols = H;
    LLP_HIP(launch_zero_rows(za, s), "zero kernel launch");
    if (out->dbias != nullptr) {
      za.p = out->dbias;
      za.ld = 1;
      za.cols = 1;
      LLP_HIP(launch_zero_rows(za, s), "zero kernel launch");
    }
  }
  if (T == 0) return LLP_OK;

  LayoutArgs la{};
  la.T = T;
  la.mask = req->layout.loss_mask;
  la.cu_seqlens = req->layout.cu_seqlens;
  la.num_seqs = req->layout.num_seqs;
  la.world = req->vocab.world;
  la.targets = req->target_ids;
  la.offset = req->vocab.offset;
  la.n_real = n_real;
  la.real_vocab = req->vocab.real_vocab;
  la.count = at<int32_t>(workspace, w.count);
  la.scored = at<int32_t>(workspace, w.scored);
  la.pos = at<int32_t>(workspace, w.pos);
  la.tloc = at<int32_t>(workspace, w.tloc);
  la.status = req->status_word;
  // Gradient, dhidden and dweight counters for each vocabulary slab (one slab unless
  // LLP_FLAG_G_SLABS splits the shard's columns).
  int32_t* qctr = at<int32_t>(workspace, w.qctr);
  la.qctr = qctr;
  la.nqctr = (int32_t)(3 * QCTR_INTS * (w.nslab > 0 ? w.nslab : 1));
  LLP_HIP(launch_layout(la, s), "layout kernel launch");

  const int ntb = (int)(w.T_cap / TILE);
  uint16_t* G = at<uint16_t>(workspace, w.G);
  uint16_t* hgT = at<uint16_t>(workspace, w.hgT);
  float* P = at<float>(workspace, w.P);
  if (n_real > 0) {
    // The dweight product's hidden operand: the scored hidden rows transposed (hgT[h][j], zero
    // past the count). G and the weight are read in place, K-major, by the other products.
    TransposeArgs th{};
    th.in = static_cast<const uint16_t*>(req->proj.hidden);
    th.ldi = req->proj.hidden_stride;
    th.idx = la.scored;
    th.count = la.count;
    th.cols = (int32_t)H;
    th.out = hgT;
    th.ldo = w.T_cap;
    LLP_HIP(launch_transpose(th, w.T_cap, s), "transpose kernel launch");

    // Vocabulary slabs in order (the whole shard is one slab by default). Each slab's G tiles
    // are written to the workspace, then read by its dhidden product (added into the fp32
    // partials after the first slab) and its dweight and dbias products, which write the
    // slab's own rows.
    const uint16_t* W = static_cast<const uint16_t*>(req->proj.weight);
    const int64_t slab_cols = w.slab_tiles * TILE;
    for (int64_t sl = 0; sl < w.nslab; ++sl) {
      const int64_t v0 = sl * slab_cols;
      const int64_t nr = n_real - v0 < slab_cols ? n_real - v0 : slab_cols;
      const int32_t nvt = (int32_t)((nr + TILE - 1) / TILE);
      int32_t* qs = qctr + 3 * QCTR_INTS * sl;

      GradArgs ga{};
      ga.W = W + v0 * req->proj.weight_stride;
      ga.ldw = req->proj.weight_stride;
      ga.h = static_cast<const uint16_t*>(req->proj.hidden);
      ga.ldh = req->proj.hidden_stride;
      ga.bias_f32 = req->proj.bias_dtype == LLP_DTYPE_F32;
      ga.bias = req->proj.bias == nullptr ? nullptr
                : ga.bias_f32 ? (const void*)(static_cast<const float*>(req->proj.bias) + v0)
                              : (const void*)(static_cast<const uint16_t*>(req->proj.bias) + v0);
      ga.H = (int32_t)H;
      ga.n_real = nr;
      ga.nvt = nvt;
      ga.ntb = ntb;
      ga.c1 = (float)(1.0 / (double)req->temperature);
      ga.count = la.count;
      ga.scored = la.scored;
      ga.tloc = la.tloc;
      ga.toff = (int32_t)v0;
      ga.lse = in->lse;
      ga.dlogp = in->dlogp;
      ga.dent = in->dentropy;
      ga.ent = in->entropy;
      ga.G = G;
      ga.ldg = w.ldg;
      ga.qctr = qs;
      ga.dbp = out->dbias != nullptr ? at<float>(workspace, w.dbp) : nullptr;
      LLP_HIP(launch_grad(ga, s), "gradient kernel launch");

      DhArgs da{};
      da.G = G;
      da.ldg = w.ldg;
      da.W = ga.W;
      da.ldw = req->proj.weight_stride;
      da.n_real = nr;
      da.H = (int32_t)H;
      da.ntm = ntb;
      da.ntn = (int32_t)((H + TILE - 1) / TILE);
      da.nsplit = DH_SPLITS;
      da.nks = (int32_t)((nr + KSTEP - 1) / KSTEP);
      da.count = la.count;
      da.P = P;
      da.pstride = w.T_cap;
      da.accumulate = sl > 0;
      da.qctr = qs + QCTR_INTS;
      LLP_HIP(launch_dh(da, s), "dhidden kernel launch");

      DwArgs wa{};
      wa.G = G;
      wa.ldg = w.ldg;
      wa.hgT = hgT;
      wa.ldk = w.T_cap;
      wa.H = (int32_t)H;
      wa.ntm = nvt;
      wa.ntn = da.ntn;
      wa.n_real = nr;
      wa.count = la.count;
      wa.dW = out->dweight + v0 * out->dweight_stride;
      wa.lddw = out->dweight_stride;
      wa.overwrite = overwrite;
      wa.qctr = qs + 2 * QCTR_INTS;
      LLP_HIP(launch_dw(wa, s), "dweight kernel launch");

      if (out->dbias != nullptr) {
        DbArgs ba{};
        ba.dbp = ga.dbp;
        ba.ldp = w.ldg;
        ba.n_real = nr;
        ba.count = la.count;
        ba.db = out->dbias + v0;
        ba.overwrite = overwrite;
        LLP_HIP(launch_dbias(ba, s), "dbias kernel launch");
      }
    }
  }
  DhReduceArgs ra{};
  ra.T = T;
  ra.H = (int32_t)H;
  ra.nsplit = n_real > 0 ? DH_SPLITS : 0;
  ra.pos = la.pos;
  ra.P = P;
  ra.pstride = w.T_cap;
  ra.dH = static_cast<uint16_t*>(out->dhidden);
  ra.ldd = out->dhidden_stride;
  LLP_HIP(launch_dh_reduce(ra, s), "dhidden reduce kernel launch");
  return LLP_OK;
}

LLP_API llp_status llp_top_p_replay(const llp_topp_request* req, const llp_partials* out,
                                    void* stream) {
  LLP_CHECK(req != nullptr && out != nullptr, LLP_ERR_INVALID_ARGUMENT, "req/out is NULL");
  llp_status st = check_partition(req->vocab);
  if (st != LLP_OK) return st;
  const int64_t T = req->num_tokens;
  LLP_CHECK(T >= 0 && T < (int64_t(1) << 31), LLP_ERR_INVALID_ARGUMENT, "num_tokens out of range");
  LLP_CHECK(req->processed_logprobs == 1, LLP_ERR_INVALID_ARGUMENT,
            "top-p replay scores processed logprobs only (processed_logprobs must be 1)");
  LLP_CHECK(req->num_replay >= 1 && req->num_replay <= LLP_MAX_REPLAY_IDS,
            LLP_ERR_INVALID_ARGUMENT, "num_replay=%d outside [1, %d]", req->num_replay,
            LLP_MAX_REPLAY_IDS);
  LLP_CHECK(req->replay_stride >= req->num_replay, LLP_ERR_INVALID_ARGUMENT,
            "replay_stride < num_replay");
  LLP_CHECK(req->logits_dtype == LLP_DTYPE_F32 || req->logits_dtype == LLP_DTYPE_BF16,
            LLP_ERR_INVALID_ARGUMENT, "logits_dtype %d is not F32 or BF16", req->logits_dtype);
  LLP_CHECK(req->logits_stride >= req->vocab.local_size, LLP_ERR_INVALID_ARGUMENT,
            "logits_stride < local_size");
  LLP_CHECK(isfinite(req->temperature) && req->temperature > 0.f, LLP_ERR_INVALID_ARGUMENT,
            "temperature must be finite and > 0");
  LLP_CHECK(out->entropy == nullptr, LLP_ERR_INVALID_ARGUMENT,
            "top-p replay produces no entropy (out.entropy must be NULL)");
  if (T > 0) {
    LLP_CHECK(req->replay_ids && req->target_ids, LLP_ERR_INVALID_ARGUMENT,
              "replay_ids and target_ids are required");
    LLP_CHECK(req->logits || local_real(req->vocab) == 0, LLP_ERR_INVALID_ARGUMENT,
              "logits is NULL");
    LLP_CHECK(out->target_logit && out->in_range && out->lse, LLP_ERR_INVALID_ARGUMENT,
              "out.target_logit, out.in_range and out.lse are required");
  }
  st = check_device();
  if (st != LLP_OK) return st;
  if (T == 0) return LLP_OK;
  ToppArgs ta{};
  ta.T = T;
  ta.logits = req->logits;
  ta.bf16 = req->logits_dtype == LLP_DTYPE_BF16;
  ta.K = req->num_replay;
  ta.lstride = req->logits_stride;
  ta.ids = req->replay_ids;
  ta.ids_stride = req->replay_stride;
  ta.targets = req->target_ids;
  ta.mask = req->loss_mask;
  ta.offset = req->vocab.offset;
  ta.n_real = local_real(req->vocab);
  ta.real_vocab = req->vocab.real_vocab;
  ta.c1 = (float)(1.0 / (double)req->temperature);
  ta.out_t = out->target_logit;
  ta.out_f = out->in_range;
  ta.out_l = out->lse;
  ta.out_p = out->logp;
  ta.status = req->status_word;
  LLP_HIP(launch_topp(ta, static_cast<hipStream_t>(stream)), "top-p replay kernel launch");
  return LLP_OK;
}

}  // extern "C"
