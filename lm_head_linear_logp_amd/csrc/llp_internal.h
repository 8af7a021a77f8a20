// llp_internal.h -- kernel argument blocks and launchers shared by the C-ABI host code and
// the HIP kernels. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "llp.h"

namespace llp {

// Number of fixed K (vocabulary) ranges the dhidden product is split into. Fixed, so that a
// row's summation order never depends on the batch.
constexpr int DH_SPLITS = 2;
constexpr int TILE = 256;  // BM = BN of every GEMM tile
// Static device scratch of llp_forward_noalloc: the forward workspace of up to this many bytes
// (T = 4096 rows over a 151936-column vocabulary need 29.2 MB).
constexpr size_t SCRATCH_BYTES = size_t(32) << 20;
constexpr int MAX_DEVICES = 64;
constexpr int KSTEP = 64;  // K depth of one pipelined GEMM step
constexpr int QCTR_INTS = 16;  // tile-queue counters per GEMM kernel launch (llp_tile.hpp)
// Vocabulary tiles per slab of G with LLP_FLAG_G_SLABS (LLP_G_SLAB_COLUMNS / TILE).
constexpr int G_SLAB_TILES = LLP_G_SLAB_COLUMNS / 256;
// Rows per workgroup of the layout scan when it takes several; up to that many rows one
// workgroup scans them all.
constexpr int64_t LAYOUT_BLOCK_ROWS = 16384;
inline int64_t layout_blocks(int64_t T) {
  return T > LAYOUT_BLOCK_ROWS ? (T + LAYOUT_BLOCK_ROWS - 1) / LAYOUT_BLOCK_ROWS : 1;
}

struct LayoutArgs {
  int64_t T;
  const uint8_t* mask;
  const int32_t* cu_seqlens;
  int32_t num_seqs;
  int32_t world;
  const int64_t* targets;
  int64_t offset, n_real, real_vocab;
  int32_t* count;   // [1 + layout_blocks(T)]: scored rows, then per layout block (if several)
  int32_t* scored;  // [T] compact index -> row
  int32_t* pos;     // [T] row -> compact index or -1
  int32_t* tloc;    // [T] compact index -> local target column or -1
  float* out_t;     // zero outputs of unscored rows (any may be null)
  uint8_t* out_f;
  float* out_l;
  float* out_e;
  float* out_p;
  int32_t* status;
  int32_t* qctr;    // tile-queue counters of the GEMM kernels of this call, zeroed here
  int32_t nqctr;
};

struct FwdArgs {
  const uint16_t* W;
  int64_t ldw;
  const uint16_t* h;
  int64_t ldh;
  const void* bias;
  int32_t bias_f32;
  int32_t H;
  int64_t n_real;
  int32_t nvt, ntb;
  float c1;
  const int32_t* count;
  const int32_t* scored;
  const int32_t* tloc;
  float* pm;
  float* ps;
  float* pq;
  float* tz;
  int64_t pstride;  // row capacity of the partial arrays (ntb * 256)
  int32_t* qctr;    // tile-queue counters (QCTR_INTS), zero at launch
  int32_t workers;  // host side: persistent workers to launch (the device's compute units)
};

struct CombineArgs {
  int32_t nvt;
  int64_t pstride;
  const int32_t* count;
  const int32_t* scored;
  const int32_t* tloc;
  const float* pm;
  const float* ps;
  const float* pq;
  const float* tz;
  float* out_t;
  uint8_t* out_f;
  float* out_l;
  float* out_e;
  float* out_p;
};

struct MergeArgs {
  int64_t T;
  int32_t world;
  const uint8_t* mask;
  const float* tl[LLP_MAX_WORLD];
  const uint8_t* flag[LLP_MAX_WORLD];
  const float* lse[LLP_MAX_WORLD];
  const float* ent[LLP_MAX_WORLD];
  float* out_p;
  float* out_l;
  float* out_e;
  int32_t* status;
};

struct ToppArgs {
  int64_t T;
  const void* logits;
  int32_t bf16;
  int32_t K;
  int64_t lstride;
  const int64_t* ids;
  int64_t ids_stride;
  const int64_t* targets;
  const uint8_t* mask;
  int64_t offset, n_real, real_vocab;
  float c1;
  float* out_t;
  uint8_t* out_f;
  float* out_l;
  float* out_p;
  int32_t* status;
};

struct LogitsArgs {
  int64_t T;
  const void* logits;
  int32_t bf16;
  int64_t ld;
  int64_t offset, n_real, real_vocab;
  int32_t world;
  const uint8_t* mask;
  const int32_t* cu_seqlens;
  int32_t num_seqs;
  const int64_t* targets;
  float c1;
  float* out_t;
  uint8_t* out_f;
  float* out_l;
  float* out_e;
  float* out_p;
  int32_t* status;
};

struct KeepArgs {
  int64_t T;
  const void* logits;
  int32_t bf16;
  int64_t lstride;
  const uint8_t* keep;
  int64_t kstride;
  int64_t offset, n_real, real_vocab;
  const uint8_t* mask;
  const int64_t* targets;
  float c1;
  float* out_t;
  uint8_t* out_f;
  float* out_l;
  float* out_p;
  int32_t* status;
};

struct GradArgs {
  const uint16_t* W;
  int64_t ldw;
  const uint16_t* h;
  int64_t ldh;
  const void* bias;
  int32_t bias_f32;
  int32_t H;
  int64_t n_real;
  int32_t nvt, ntb;
  float c1;
  const int32_t* count;
  const int32_t* scored;
  const int32_t* tloc;
  int32_t toff;     // local column of the weight's first row (a vocabulary slab's first column)
  const float* lse;
  const float* dlogp;
  const float* dent;
  const float* ent;
  uint16_t* G;
  int64_t ldg;
  int32_t* qctr;    // tile-queue counters (QCTR_INTS), zero at launch
  float* dbp;       // bias-gradient partials [token block][ldg] (column sums of each G tile),
                    // or null when the request has no bias
};

struct DhArgs {
  const uint16_t* G;
  int64_t ldg;
  const uint16_t* W;  // the shard's weight rows (K-major operand of dhidden = G W)
  int64_t ldw;
  int64_t n_real;
  int32_t H;
  int32_t ntm, ntn, nsplit, nks;
  const int32_t* count;
  float* P;
  int64_t pstride;  // rows per split
  int32_t accumulate;  // 0: P = the product; 1: P += the product (later vocabulary slabs)
  int32_t* qctr;    // tile-queue counters (QCTR_INTS), zero at launch
};

struct DhReduceArgs {
  int64_t T;
  int32_t H;
  int32_t nsplit;
  const int32_t* pos;
  const float* P;
  int64_t pstride;
  uint16_t* dH;
  int64_t ldd;
};

struct DwArgs {
  const uint16_t* G;  // [scored row][local vocabulary], K-major operand of dweight = G^T hg
  int64_t ldg;
  const uint16_t* hgT;
  int64_t ldk;  // row stride of hgT (the scored-row capacity)
  int32_t H;
  int32_t ntm, ntn;
  int64_t n_real;
  const int32_t* count;
  float* dW;
  int64_t lddw;
  int32_t overwrite;  // 1: dW = the product (no read of dW); 0: dW += the product
  int32_t* qctr;    // tile-queue counters (QCTR_INTS), zero at launch
};

struct ZeroArgs {
  float* p;
  int64_t ld;
  int64_t r0, r1;  // rows [r0, r1)
  int64_t cols;
};

struct TransposeArgs {
  const uint16_t* in;
  int64_t ldi;
  const int32_t* idx;    // row gather list or null
  const int32_t* count;  // number of valid rows on the device, or null (use nvalid)
  int64_t nvalid;
  int32_t cols;          // columns of `in` read (multiple of 64)
  uint16_t* out;
  int64_t ldo;
};

struct DbArgs {
  const float* dbp;  // [token block][ldp] partials of the gradient tiles
  int64_t ldp;
  int64_t n_real;
  const int32_t* count;
  float* db;
  int32_t overwrite;  // 1: db = the sum; 0: db += the sum
};

hipError_t launch_layout(const LayoutArgs& a, hipStream_t s);
hipError_t launch_fwd(const FwdArgs& a, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, int64_t T_cap, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_topp(const ToppArgs& a, hipStream_t s);
hipError_t launch_grad(const GradArgs& a, hipStream_t s);
hipError_t launch_dh(const DhArgs& a, hipStream_t s);
hipError_t launch_dh_reduce(const DhReduceArgs& a, hipStream_t s);
hipError_t launch_dw(const DwArgs& a, hipStream_t s);
hipError_t launch_transpose(const TransposeArgs& a, int64_t rows, hipStream_t s);
hipError_t launch_dbias(const DbArgs& a, hipStream_t s);
hipError_t launch_zero_rows(const ZeroArgs& a, hipStream_t s);
hipError_t launch_logits(const LogitsArgs& a, hipStream_t s);
hipError_t launch_keep(const KeepArgs& a, hipStream_t s);
hipError_t probe_kernels();
// Looks up this device's copy of the static scratch (the current device must be `device`);
// idempotent. Called under the library's open lock.
hipError_t scratch_init(int device);
// The device address of that copy, or null before scratch_init succeeded on the device.
void* scratch_address(int device);

}  // namespace llp
