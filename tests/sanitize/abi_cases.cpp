// abi_cases.cpp -- runs the C ABI's host code (built with the sanitizers, on the stub runtime
// of hip_stub.cpp) through malformed requests, which must be refused with the documented
// status, and well-formed ones for every entry point, whose launch sequences must address only
// the exactly sized buffers handed in. Exit status 0 when every case behaves; a sanitizer
// report aborts the run.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <functional>
#include <string>
#include <vector>

#include "llp.h"

extern "C" int64_t llp_stub_launches();

static int g_fail = 0, g_cases = 0;

static void expect(const char* name, llp_status got, llp_status want) {
  ++g_cases;
  if (got != want) {
    ++g_fail;
    fprintf(stderr, "FAIL %s: status %d, expected %d (%s)\n", name, (int)got, (int)want,
            llp_last_error());
  }
}

// Exactly sized host buffers: posix_memalign with the exact byte count, so that the address
// sanitizer poisons everything past the requested size (the stub launchers touch extents).
struct Buf {
  std::vector<void*> keep;
  void* get(size_t bytes, size_t align = 256) {
    if (bytes == 0) return nullptr;
    void* p = nullptr;
    if (posix_memalign(&p, align < sizeof(void*) ? sizeof(void*) : align, bytes) != 0) abort();
    memset(p, 0, bytes);
    keep.push_back(p);
    return p;
  }
  ~Buf() {
    for (void* p : keep) free(p);
  }
};

struct Shape {
  int64_t T, H, V, Vr, off, loc;
  int32_t rank, world;
};

static llp_request make_request(Buf& b, const Shape& s, bool bias_f32, bool bias, bool mask,
                                bool cu) {
  llp_request r;
  memset(&r, 0, sizeof(r));
  r.proj.hidden = b.get((size_t)s.T * s.H * 2, 16);
  r.proj.hidden_stride = s.H;
  r.proj.weight = b.get((size_t)s.loc * s.H * 2, 16);
  r.proj.weight_stride = s.H;
  if (bias) {
    r.proj.bias = b.get((size_t)s.loc * (bias_f32 ? 4 : 2), 16);
    r.proj.bias_dtype = bias_f32 ? LLP_DTYPE_F32 : LLP_DTYPE_BF16;
  }
  r.proj.hidden_size = s.H;
  r.vocab.offset = s.off;
  r.vocab.local_size = s.loc;
  r.vocab.real_vocab = s.Vr;
  r.vocab.padded_vocab = s.V;
  r.vocab.rank = s.rank;
  r.vocab.world = s.world;
  r.layout.num_tokens = s.T;
  if (mask) r.layout.loss_mask = (const uint8_t*)b.get((size_t)s.T, 1);
  if (cu) {
    r.layout.num_seqs = 3;
    r.layout.cu_seqlens = (const int32_t*)b.get(4 * 4, 4);
  }
  r.target_ids = (const int64_t*)b.get((size_t)s.T * 8, 8);
  r.temperature = 0.7f;
  r.flags = LLP_FLAG_WANT_ENTROPY;
  r.status_word = (int32_t*)b.get(4, 4);
  return r;
}

static llp_partials make_partials(Buf& b, int64_t T, bool ent, bool logp) {
  llp_partials o;
  o.target_logit = (float*)b.get((size_t)T * 4, 4);
  o.in_range = (uint8_t*)b.get((size_t)T, 1);
  o.lse = (float*)b.get((size_t)T * 4, 4);
  o.entropy = ent ? (float*)b.get((size_t)T * 4, 4) : nullptr;
  o.logp = logp ? (float*)b.get((size_t)T * 4, 4) : nullptr;
  return o;
}

static void forward_case(const char* name, const Shape& s, bool bias, bool bias_f32, bool mask,
                         bool cu) {
  Buf b;
  llp_request r = make_request(b, s, bias_f32, bias, mask, cu);
  llp_partials o = make_partials(b, s.T, true, true);
  size_t ws = 0;
  expect(name, llp_workspace_bytes(&r, LLP_OP_FORWARD, &ws), LLP_OK);
  void* w = b.get(ws, 256);
  expect(name, llp_forward(&r, &o, w, ws, nullptr), LLP_OK);
  if (ws <= ((size_t)32 << 20)) expect(name, llp_forward_noalloc(&r, &o, nullptr), LLP_OK);
  // One byte less workspace is refused.
  if (ws > 0) expect(name, llp_forward(&r, &o, w, ws - 1, nullptr), LLP_ERR_INVALID_ARGUMENT);
}

static void backward_case(const char* name, const Shape& s, bool bias, bool dent, bool overwrite,
                          bool slabs = false) {
  Buf b;
  llp_request r = make_request(b, s, true, bias, true, false);
  if (overwrite) r.flags |= LLP_FLAG_OVERWRITE_GRADS;
  if (slabs) {
    // G held one vocabulary slab at a time: a smaller workspace than the default mode's.
    size_t whole = 0, slab = 0;
    expect(name, llp_workspace_bytes(&r, LLP_OP_BACKWARD, &whole), LLP_OK);
    r.flags |= LLP_FLAG_G_SLABS;
    expect(name, llp_workspace_bytes(&r, LLP_OP_BACKWARD, &slab), LLP_OK);
    expect(name, slab < whole ? LLP_OK : LLP_ERR_INTERNAL, LLP_OK);
  }
  llp_bwd_in in;
  in.lse = (const float*)b.get((size_t)s.T * 4, 4);
  in.dlogp = (const float*)b.get((size_t)s.T * 4, 4);
  in.dentropy = dent ? (const float*)b.get((size_t)s.T * 4, 4) : nullptr;
  in.entropy = dent ? (const float*)b.get((size_t)s.T * 4, 4) : nullptr;
  llp_bwd_out out;
  out.dhidden = b.get((size_t)s.T * s.H * 2, 16);
  out.dhidden_stride = s.H;
  out.dweight = (float*)b.get((size_t)s.loc * s.H * 4, 16);
  out.dweight_stride = s.H;
  out.dbias = bias ? (float*)b.get((size_t)s.loc * 4, 16) : nullptr;
  size_t ws = 0;
  expect(name, llp_workspace_bytes(&r, LLP_OP_BACKWARD, &ws), LLP_OK);
  void* w = b.get(ws, 256);
  expect(name, llp_backward(&r, &in, &out, w, ws, nullptr), LLP_OK);
}

static void replay_cases() {
  for (int bf16 = 0; bf16 < 2; ++bf16)
    for (const Shape& s : {Shape{37, 0, 1024, 1000, 0, 1024, 0, 1},
                           Shape{300, 0, 1024, 1000, 768, 256, 3, 4},
                           Shape{5, 0, 1024, 1000, 0, 0, 0, 2}}) {
      Buf b;
      const int64_t es = bf16 ? 2 : 4;
      llp_topp_request q;
      memset(&q, 0, sizeof(q));
      q.logits = b.get((size_t)s.T * s.loc * es + 16, 16);
      q.logits_dtype = bf16 ? LLP_DTYPE_BF16 : LLP_DTYPE_F32;
      q.num_replay = 64;
      q.logits_stride = s.loc;
      q.num_tokens = s.T;
      q.vocab = {s.off, s.loc, s.Vr, s.V, s.rank, s.world};
      q.replay_ids = (const int64_t*)b.get((size_t)s.T * 64 * 8, 8);
      q.replay_stride = 64;
      q.target_ids = (const int64_t*)b.get((size_t)s.T * 8, 8);
      q.loss_mask = (const uint8_t*)b.get((size_t)s.T, 1);
      q.temperature = 0.7f;
      q.processed_logprobs = 1;
      llp_partials o = make_partials(b, s.T, false, true);
      expect("top_p_replay", llp_top_p_replay(&q, &o, nullptr), LLP_OK);
      q.num_replay = 65;
      expect("top_p_replay K=65", llp_top_p_replay(&q, &o, nullptr), LLP_ERR_INVALID_ARGUMENT);
      q.num_replay = 64;
      q.processed_logprobs = 0;
      expect("top_p_replay raw", llp_top_p_replay(&q, &o, nullptr), LLP_ERR_INVALID_ARGUMENT);

      llp_logits_request lr;
      memset(&lr, 0, sizeof(lr));
      const int64_t ld = (s.loc * es + 15) / 16 * 16 / es;
      lr.logits = b.get((size_t)s.T * (ld > 0 ? ld : 1) * es, 16);
      lr.logits_dtype = q.logits_dtype;
      lr.logits_stride = ld;
      lr.vocab = q.vocab;
      lr.layout.num_tokens = s.T;
      lr.layout.loss_mask = q.loss_mask;
      lr.target_ids = q.target_ids;
      lr.temperature = 0.7f;
      lr.flags = LLP_FLAG_WANT_ENTROPY;
      llp_partials o2 = make_partials(b, s.T, true, true);
      expect("forward_logits", llp_forward_logits(&lr, &o2, nullptr), LLP_OK);

      llp_keep_mask_request kr;
      memset(&kr, 0, sizeof(kr));
      kr.logits = lr.logits;
      kr.logits_dtype = lr.logits_dtype;
      kr.processed_logprobs = 1;
      kr.logits_stride = ld;
      const int64_t kst = (s.loc + 15) / 16 * 16;
      kr.keep_mask = (const uint8_t*)b.get((size_t)s.T * (kst > 0 ? kst : 16), 16);
      kr.keep_stride = kst;
      kr.num_tokens = s.T;
      kr.vocab = q.vocab;
      kr.target_ids = q.target_ids;
      kr.loss_mask = q.loss_mask;
      kr.temperature = 0.7f;
      llp_partials o3 = make_partials(b, s.T, false, true);
      expect("keep_mask_replay", llp_keep_mask_replay(&kr, &o3, nullptr), LLP_OK);
    }
}

static void merge_cases() {
  for (int world : {1, 2, 5, 64}) {
    Buf b;
    const int64_t T = 333;
    std::vector<llp_partials> parts;
    for (int r = 0; r < world; ++r) parts.push_back(make_partials(b, T, true, false));
    llp_final_out out{(float*)b.get(T * 4, 4), (float*)b.get(T * 4, 4), (float*)b.get(T * 4, 4)};
    const uint8_t* mask = (const uint8_t*)b.get(T, 1);
    expect("merge", llp_merge(world, parts.data(), T, mask, &out, (int32_t*)b.get(4, 4), nullptr),
           LLP_OK);
  }
  Buf b;
  llp_partials p = make_partials(b, 8, true, false);
  llp_final_out out{(float*)b.get(32, 4), (float*)b.get(32, 4), nullptr};
  std::vector<llp_partials> many(65, p);
  expect("merge world 65", llp_merge(65, many.data(), 8, nullptr, &out, nullptr, nullptr),
         LLP_ERR_INVALID_ARGUMENT);
  expect("merge T<0", llp_merge(1, &p, -1, nullptr, &out, nullptr, nullptr),
         LLP_ERR_INVALID_ARGUMENT);
}

static void malformed_cases() {
  const Shape s{64, 256, 1024, 1000, 0, 1024, 0, 1};
  struct Bad {
    const char* name;
    std::function<void(llp_request&)> f;
    llp_status want;
  };
  std::vector<Bad> bad = {
      {"negative T", [](llp_request& r) { r.layout.num_tokens = -1; }, LLP_ERR_INVALID_ARGUMENT},
      {"H not multiple of 64", [](llp_request& r) { r.proj.hidden_size = 200; r.proj.hidden_stride = 200; r.proj.weight_stride = 200; }, LLP_ERR_UNSUPPORTED},
      {"hidden stride < H", [](llp_request& r) { r.proj.hidden_stride = 255; }, LLP_ERR_INVALID_ARGUMENT},
      {"weight stride odd", [](llp_request& r) { r.proj.weight_stride = 257; }, LLP_ERR_INVALID_ARGUMENT},
      {"hidden misaligned", [](llp_request& r) { r.proj.hidden = (const char*)r.proj.hidden + 2; }, LLP_ERR_INVALID_ARGUMENT},
      {"weight NULL", [](llp_request& r) { r.proj.weight = nullptr; }, LLP_ERR_INVALID_ARGUMENT},
      {"targets NULL", [](llp_request& r) { r.target_ids = nullptr; }, LLP_ERR_INVALID_ARGUMENT},
      {"tau zero", [](llp_request& r) { r.temperature = 0.f; }, LLP_ERR_INVALID_ARGUMENT},
      {"tau nan", [](llp_request& r) { r.temperature = __builtin_nanf(""); }, LLP_ERR_INVALID_ARGUMENT},
      {"tau inf", [](llp_request& r) { r.temperature = __builtin_inff(); }, LLP_ERR_INVALID_ARGUMENT},
      {"real > padded", [](llp_request& r) { r.vocab.real_vocab = 1025; }, LLP_ERR_INVALID_ARGUMENT},
      {"world1 partial shard", [](llp_request& r) { r.vocab.local_size = 1000; }, LLP_ERR_INVALID_ARGUMENT},
      {"rank >= world", [](llp_request& r) { r.vocab.world = 4; r.vocab.rank = 4; r.vocab.local_size = 256; }, LLP_ERR_INVALID_ARGUMENT},
      {"world too big", [](llp_request& r) { r.vocab.world = 65; }, LLP_ERR_INVALID_ARGUMENT},
      {"bad bias dtype", [](llp_request& r) { r.proj.bias = r.proj.weight; r.proj.bias_dtype = 7; }, LLP_ERR_INVALID_ARGUMENT},
      {"unknown flag", [](llp_request& r) { r.flags = 8; }, LLP_ERR_INVALID_ARGUMENT},
      {"T too large", [](llp_request& r) { r.layout.num_tokens = int64_t(1) << 23; }, LLP_ERR_UNSUPPORTED},
      {"hidden bytes 2^31", [](llp_request& r) { r.layout.num_tokens = int64_t(1) << 22; r.proj.hidden_stride = 256; }, LLP_ERR_UNSUPPORTED},
      {"T * stride overflow", [](llp_request& r) { r.layout.num_tokens = (int64_t(1) << 23) - 256; r.proj.hidden_stride = (int64_t(1) << 23) - 8; }, LLP_ERR_UNSUPPORTED},
      {"weight stride 2^23", [](llp_request& r) { r.proj.weight_stride = int64_t(1) << 23; }, LLP_ERR_UNSUPPORTED},
      {"padded_vocab huge", [](llp_request& r) { r.vocab.padded_vocab = int64_t(1) << 40; r.vocab.local_size = int64_t(1) << 40; r.vocab.real_vocab = int64_t(1) << 40; }, LLP_ERR_UNSUPPORTED},
      {"offset + local overflow", [](llp_request& r) { r.vocab.world = 2; r.vocab.offset = INT64_MAX - 5; r.vocab.local_size = 100; }, LLP_ERR_INVALID_ARGUMENT},
      {"negative num_seqs", [](llp_request& r) { r.layout.cu_seqlens = (const int32_t*)r.target_ids; r.layout.num_seqs = -1; }, LLP_ERR_INVALID_ARGUMENT},
  };
  for (const Bad& c : bad) {
    Buf b;
    llp_request r = make_request(b, s, false, false, false, false);
    c.f(r);
    llp_partials o = make_partials(b, s.T, true, true);
    size_t ws = 0;
    const llp_status st = llp_workspace_bytes(&r, LLP_OP_FORWARD, &ws);
    expect(c.name, st, c.want);
    std::vector<unsigned char> w(1 << 16);
    expect(c.name, llp_forward(&r, &o, w.data(), 0, nullptr), c.want);
    expect(c.name, llp_forward_noalloc(&r, &o, nullptr), c.want);
    llp_bwd_in in{o.lse, o.lse, nullptr, nullptr};
    llp_bwd_out out{b.get(s.T * s.H * 2, 16), s.H, (float*)b.get(s.loc * s.H * 4, 16), s.H, nullptr};
    expect(c.name, llp_backward(&r, &in, &out, w.data(), 0, nullptr), c.want);
  }
  {  // NULL request / outputs
    expect("NULL request", llp_forward(nullptr, nullptr, nullptr, 0, nullptr), LLP_ERR_INVALID_ARGUMENT);
    expect("NULL workspace_bytes", llp_workspace_bytes(nullptr, LLP_OP_FORWARD, nullptr), LLP_ERR_INVALID_ARGUMENT);
    Buf b;
    llp_request r = make_request(b, s, false, false, false, false);
    size_t ws = 0;
    expect("bad op", llp_workspace_bytes(&r, 9, &ws), LLP_ERR_INVALID_ARGUMENT);
    expect("NULL bytes", llp_workspace_bytes(&r, LLP_OP_FORWARD, nullptr), LLP_ERR_INVALID_ARGUMENT);
    llp_partials o = make_partials(b, s.T, true, true);
    o.lse = nullptr;
    expect("forward NULL lse", llp_forward(&r, &o, nullptr, 1 << 30, nullptr), LLP_ERR_INVALID_ARGUMENT);
    expect("noalloc too large", [&] {
      llp_request big = r;
      big.layout.num_tokens = 4609;
      big.vocab = {0, 151936, 151669, 151936, 0, 1};
      return llp_forward_noalloc(&big, &o, nullptr);
    }(), LLP_ERR_UNSUPPORTED);
  }
}

int main() {
  llp_info info;
  expect("open", llp_open(0, &info), LLP_OK);
  expect("open other device", llp_open(1, &info), LLP_ERR_INVALID_ARGUMENT);
  malformed_cases();
  // Forward shapes: ragged rows and vocabulary, bias modes, masks, packing, shards, an empty
  // shard, padding only, no rows.
  forward_case("fwd small", {64, 256, 1024, 1000, 0, 1024, 0, 1}, false, false, false, false);
  forward_case("fwd ragged bias f32", {700, 512, 3072, 3000, 0, 3072, 0, 1}, true, true, true, true);
  forward_case("fwd ragged bias bf16", {1, 64, 300, 257, 0, 300, 0, 1}, true, false, true, false);
  forward_case("fwd shard", {513, 128, 4096, 3500, 1024, 1024, 1, 4}, true, true, true, false);
  forward_case("fwd last shard", {257, 128, 4096, 3500, 3072, 1024, 3, 4}, false, false, true, false);
  forward_case("fwd padding-only shard", {100, 64, 4096, 3000, 3072, 1024, 3, 4}, false, false, false, false);
  forward_case("fwd empty shard", {100, 64, 4096, 3000, 4096, 0, 4, 5}, false, false, false, false);
  forward_case("fwd no rows", {0, 64, 1024, 1000, 0, 1024, 0, 1}, false, false, false, false);
  backward_case("bwd", {300, 256, 1024, 1000, 0, 1024, 0, 1}, false, false, false);
  backward_case("bwd bias dentropy overwrite", {700, 512, 3072, 3000, 0, 3072, 0, 1}, true, true, true);
  backward_case("bwd shard", {129, 64, 4096, 3500, 3072, 1024, 3, 4}, true, false, true);
  backward_case("bwd padding-only shard", {64, 64, 4096, 3000, 3072, 1024, 3, 4}, true, false, true);
  backward_case("bwd empty shard", {64, 64, 4096, 3000, 4096, 0, 4, 5}, false, false, true);
  backward_case("bwd no rows overwrite", {0, 64, 1024, 1000, 0, 1024, 0, 1}, true, false, true);
  backward_case("bwd slabs", {130, 64, 70144, 70000, 0, 70144, 0, 1}, true, true, true, true);
  backward_case("bwd slabs accumulate", {257, 64, 70144, 70000, 0, 70144, 0, 1}, true, false,
                false, true);
  backward_case("bwd slabs shard", {64, 64, 151936, 151669, 113952, 37984, 3, 4}, true, false,
                true, true);
  replay_cases();
  merge_cases();
  printf("%d cases, %d failed, %lld launches\n", g_cases, g_fail, (long long)llp_stub_launches());
  return g_fail == 0 ? 0 : 1;
}
