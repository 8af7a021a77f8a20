// llp_kernels.hip -- HIP kernels of the fused linear log-prob operator for gfx950 and their
// launchers. Every reduction has a fixed order that depends only on vocabulary / K position,
// never on a row's position in the batch, and no float atomics are used: results are
// bitwise reproducible and independent of how rows are packed.
//
// Sources: [CUDA provider] "feat(rl-kernel): add CUDA linear logp provider integration",
// [ROCm provider] "feat(rl-kernel): add ROCm linear logp provider integration",
// [top-p replay] "Perf/cuda compact top p replay".
#include "llp_internal.h"
#include "llp_tile.hpp"

#include <math.h>

namespace llp {

// ------------------------------------------------------------------------------------
// Layout and mask indexing. A workgroup scans the loss mask in order (16 rows per thread and
// pass) and writes the compact list of scored rows, each row's compact index (-1 when
// unscored), the target's local column (-1 when outside this shard's real columns), zero
// outputs for unscored rows, and status bits ([CUDA provider, "Summary"]: the framework keeps
// token layout and masking; the operator scores unmasked rows only). Up to LAYOUT_BLOCK rows
// one workgroup does it all; beyond, workgroup b takes rows [b, b + 1) * LAYOUT_BLOCK and
// starts its compact indices after the scored rows of the blocks before it, counted by
// k_layout_count in a launch of its own (no workgroup waits for another). Either way row t's
// compact index is the number of scored rows before t.
// count[0] = the number of scored rows; count[1 + b] = block b's (multi-block launch only).
// ------------------------------------------------------------------------------------
constexpr int LAYOUT_THREADS = 1024, LAYOUT_ROWS = 16;   // rows per thread per pass
constexpr int64_t LAYOUT_BLOCK = (int64_t)LAYOUT_THREADS * LAYOUT_ROWS;
static_assert(LAYOUT_BLOCK == LAYOUT_BLOCK_ROWS, "layout block shared with the host");

__device__ __forceinline__ bool layout_scored(const LayoutArgs& a, int64_t t) {
  return t < a.T && (a.mask == nullptr || a.mask[t] != 0);
}

__global__ __launch_bounds__(LAYOUT_THREADS) void k_layout_count(LayoutArgs a) {
  __shared__ int wsum[LAYOUT_THREADS / 64];
  const int64_t t0 = (int64_t)blockIdx.x * LAYOUT_BLOCK + (int64_t)threadIdx.x * LAYOUT_ROWS;
  int cnt = 0;
#pragma unroll
  for (int k = 0; k < LAYOUT_ROWS; ++k) cnt += layout_scored(a, t0 + k) ? 1 : 0;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    int tot = 0;
    for (int w = 0; w < LAYOUT_THREADS / 64; ++w) tot += wsum[w];
    a.count[1 + blockIdx.x] = tot;
  }
}

__global__ __launch_bounds__(LAYOUT_THREADS) void k_layout(LayoutArgs a) {
  __shared__ int wsum[LAYOUT_THREADS / 64];
  __shared__ int carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int blk = blockIdx.x;
  int status = 0;
  if (wave == 0) {
    // Scored rows of the blocks before this one (integer sums: exact in any order).
    int c = 0;
    for (int b = lane; b < blk; b += 64) c += a.count[1 + b];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
    if (lane == 0) carry_s = c;
  }
  // The tile-queue counters of the GEMM kernels that follow on this stream start at 0.
  if (blk == 0)
    for (int i = tid; i < a.nqctr; i += LAYOUT_THREADS) a.qctr[i] = 0;
  __syncthreads();
  // One workgroup: every pass; several: this block's one pass.
  const int64_t first = (int64_t)blk * LAYOUT_BLOCK;
  const int64_t end = gridDim.x == 1 ? a.T : first + LAYOUT_BLOCK;
  // Each pass covers LAYOUT_THREADS * LAYOUT_ROWS rows; thread tid takes LAYOUT_ROWS
  // consecutive ones. Its scored rows get consecutive compact indices after those of all
  // lower threads (an exclusive scan of the per-thread counts), so the compaction keeps row
  // order, as a serial scan would.
  for (int64_t base = first; base < end && base < a.T; base += LAYOUT_BLOCK) {
    const int64_t t0 = base + (int64_t)tid * LAYOUT_ROWS;
    uint32_t bits = 0;
#pragma unroll
    for (int k = 0; k < LAYOUT_ROWS; ++k)
      if (layout_scored(a, t0 + k)) bits |= 1u << k;
    const int cnt = __popc(bits);
    int incl = cnt;  // inclusive scan over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int pre = carry_s;
    for (int w = 0; w < wave; ++w) pre += wsum[w];
    int j = pre + incl - cnt;
#pragma unroll
    for (int k = 0; k < LAYOUT_ROWS; ++k) {
      const int64_t t = t0 + k;
      if (t >= a.T) continue;
      const bool sc = (bits >> k) & 1u;
      a.pos[t] = sc ? j : -1;
      if (sc) {
        a.scored[j] = (int)t;
        const int64_t tg = a.targets[t];
        const bool valid = tg >= 0 && tg < a.real_vocab;
        if (!valid) status |= LLP_STATUS_TARGET_OUT_OF_RANGE;
        const int64_t loc = tg - a.offset;
        const bool hit = valid && loc >= 0 && loc < a.n_real;
        a.tloc[j] = hit ? (int)loc : -1;
        if (!hit && a.world == 1) status |= LLP_STATUS_TARGET_NOT_FOUND;
        ++j;
      } else {
        if (a.out_t) a.out_t[t] = 0.f;
        if (a.out_f) a.out_f[t] = 0;
        if (a.out_l) a.out_l[t] = 0.f;
        if (a.out_e) a.out_e[t] = 0.f;
        if (a.out_p) a.out_p[t] = 0.f;
      }
    }
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int w = 0; w < LAYOUT_THREADS / 64; ++w) tot += wsum[w];
      carry_s += tot;
    }
    __syncthreads();
  }
  if (blk == gridDim.x - 1 && tid == 0) a.count[0] = carry_s;
  if (blk == 0 && a.cu_seqlens != nullptr) {
    for (int i = tid; i <= a.num_seqs; i += LAYOUT_THREADS) {
      const int c = a.cu_seqlens[i];
      if (i == 0 && c != 0) status |= LLP_STATUS_LAYOUT_INVALID;
      if (i == a.num_seqs && (int64_t)c != a.T) status |= LLP_STATUS_LAYOUT_INVALID;
      if (i < a.num_seqs && a.cu_seqlens[i + 1] < c) status |= LLP_STATUS_LAYOUT_INVALID;
    }
  }
  if (status && a.status) atomicOr(a.status, status);
}

// ------------------------------------------------------------------------------------
// Fused forward tile: z = (h W^T + b) * (1/tau) for 256 vocabulary columns x 256 scored
// rows, then per row of the tile the max m, s = sum exp(z - m) and q = sum exp(z - m) (z - m)
// log2(e), plus the target logit when the target column lies in the tile. Columns at or
// past the shard's real vocabulary are excluded ([CUDA provider, "Megatron integration"]:
// real/padded vocabulary sizes). The [T, V] logits never leave registers.
// MFMA operand A = weight rows (vocabulary, M), B = hidden rows (tokens, N): each lane owns
// one token column, so the per-row reductions run down its own registers first.
// ------------------------------------------------------------------------------------
// The bias enters as the accumulators' starting value: z * tau = bias + h.W^T comes straight
// out of the MFMAs, so neither epilogue reads the bias, and every bias mode runs the no-bias
// epilogue with its register footprint. The forward and the gradient tile start the same way,
// so both see the same z.
//
// Bias of this lane's 16 accumulator rows of the 32-row block at vb: rows
// vb + 8g + 4(lane/32) + 0..3 for g = 0..3 (mfma_row), i.e. four runs of four consecutive
// rows, each read with one vector load (the bias is 16-byte aligned for fp32, 8-byte for
// bf16). Rows at or past n_real (only in the shard's last tile) read as 0.
template <bool F32>
__device__ __forceinline__ void bias16(const void* bias, int vb, int lane, int64_t n_real,
                                       float (&b)[16]) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int v = vb + 8 * g + 4 * (lane >> 5);
    if (v + 3 < n_real) {
      if constexpr (F32) {
        const float4 x = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(bias) + v);
        b[4 * g] = x.x;
        b[4 * g + 1] = x.y;
        b[4 * g + 2] = x.z;
        b[4 * g + 3] = x.w;
      } else {
        const uint2 x = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(bias) + v);
        b[4 * g] = __builtin_bit_cast(float, x.x << 16);
        b[4 * g + 1] = __builtin_bit_cast(float, x.x & 0xFFFF0000u);
        b[4 * g + 2] = __builtin_bit_cast(float, x.y << 16);
        b[4 * g + 3] = __builtin_bit_cast(float, x.y & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float x = 0.f;
        if (v + u < n_real)
          x = F32 ? reinterpret_cast<const float*>(bias)[v + u]
                  : bf16_to_f32(reinterpret_cast<const uint16_t*>(bias)[v + u]);
        b[4 * g + u] = x;
      }
    }
  }
}

// Starting accumulators of a vocabulary x token tile at v0: each lane's rows get their bias (the
// same for all its token blocks).
template <bool F32, int NFB>
__device__ __forceinline__ void bias_acc(f32x16 (&acc)[4][NFB], const void* bias, int v0,
                                         int64_t n_real) {
  const int lane = threadIdx.x & 63, wm = (threadIdx.x >> 6) & 1;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    float b[16];
    bias16<F32>(bias, v0 + wm * 128 + mi * 32, lane, n_real, b);
#pragma unroll
    for (int ni = 0; ni < NFB; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = b[r];
  }
}

// The same, or 0 without a bias (mode chosen at run time).
template <int NFB>
__device__ __forceinline__ void init_acc(f32x16 (&acc)[4][NFB], const void* bias, bool bias_f32,
                                         int v0, int64_t n_real) {
  if (bias == nullptr) zero_acc(acc);
  else if (bias_f32) bias_acc<true, NFB>(acc, bias, v0, n_real);
  else bias_acc<false, NFB>(acc, bias, v0, n_real);
}

constexpr int BIAS_NONE = 0, BIAS_BF16 = 1, BIAS_F32 = 2;

// NFB = 4: 4 waves (2 x 2) of 128 vocabulary columns x 128 tokens; NFB = 2: 8 waves (2 x 4)
// of 128 x 64. Either way a token's values are reduced in the same order: down the lane's
// 64 values of its wave's 128 columns (mi, r), the lane pair, then the two column halves.
template <bool TAIL, int NFB>
__device__ __forceinline__ void fwd_epilogue(const f32x16 (&acc)[4][NFB], const FwdArgs& a, int vt,
                                             int v0, int j0, int Ts, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  constexpr int TW = 32 * NFB;  // tokens per wave
  const int vbase = v0 + wm * 128;
  // red: [6][256] in LDS: max0 max1 s0 s1 q0 q1. The exchange between waves goes through LDS
  // only, so the barriers wait for LDS alone (DMA loads of a next tile may be in flight).
  // Pass 1: per-token max of x over this lane's 64 columns, the lane pair (l, l^32) and the two
  // waves holding the tile's two column halves. z = x * c1 with c1 > 0 and rounding is
  // monotonic, so fl(max x * c1) is the max of z.
  float mx[NFB];
#pragma unroll
  for (int ni = 0; ni < NFB; ++ni) mx[ni] = -INFINITY;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int ni = 0; ni < NFB; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = acc[mi][ni][r];
        if (TAIL && vbase + mi * 32 + mfma_row(r, lane) >= a.n_real) x = -INFINITY;
        mx[ni] = fmaxf(mx[ni], x);
      }
  }
#pragma unroll
  for (int ni = 0; ni < NFB; ++ni) {
    mx[ni] = fmaxf(mx[ni], __shfl_xor(mx[ni], 32));
    if (lane < 32) red[wm * 256 + wn * TW + ni * 32 + lane] = mx[ni];
  }
  dma::lds_barrier();
  // Pass 2: s = sum 2^d2, q = sum 2^d2 * d2 with d2 = (z - M) log2(e) = x c1 log2(e) - M log2(e).
  const float c1l = a.c1 * kLog2e;
  float ml[NFB];
#pragma unroll
  for (int ni = 0; ni < NFB; ++ni) {
    const int tn = wn * TW + ni * 32 + (lane & 31);
    mx[ni] = fmaxf(red[tn], red[256 + tn]) * a.c1;
    ml[ni] = mx[ni] * kLog2e;
  }
  float sv[NFB], qv[NFB];
#pragma unroll
  for (int ni = 0; ni < NFB; ++ni) sv[ni] = qv[ni] = 0.f;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int ni = 0; ni < NFB; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float d2 = fmaf(acc[mi][ni][r], c1l, -ml[ni]);
        // Excluded column: 2^-1e30 = 0 and 0 * -1e30 = 0.
        if (TAIL && vbase + mi * 32 + mfma_row(r, lane) >= a.n_real) d2 = -1e30f;
        const float e = __builtin_amdgcn_exp2f(d2);
        sv[ni] += e;
        qv[ni] = fmaf(e, d2, qv[ni]);
      }
  }
#pragma unroll
  for (int ni = 0; ni < NFB; ++ni) {
    // (x + y) == (y + x): both lanes of a pair hold the same sum.
    sv[ni] += __shfl_xor(sv[ni], 32);
    qv[ni] += __shfl_xor(qv[ni], 32);
    if (lane < 32) {
      const int tn = wn * TW + ni * 32 + lane;
      red[512 + wm * 256 + tn] = sv[ni];
      red[1024 + wm * 256 + tn] = qv[ni];
    }
  }
  dma::lds_barrier();
#pragma unroll
  for (int ni = 0; ni < NFB; ++ni) {
    const int tn = wn * TW + ni * 32 + (lane & 31);
    const int j = j0 + tn;
    if (wm == 0 && lane < 32 && j < Ts) {
      const int64_t o = (int64_t)vt * a.pstride + j;
      a.pm[o] = mx[ni];
      a.ps[o] = red[512 + tn] + red[768 + tn];
      a.pq[o] = red[1024 + tn] + red[1280 + tn];
    }
    // Target logit: the one lane holding column tloc[j] copies its z (rare: skipped unless
    // some lane of the wave holds a target).
    const int tl = (j < Ts) ? a.tloc[j] - vbase : -1;
    const bool mine = tl >= 0 && tl < 128 && (((tl & 31) >> 2) & 1) == (lane >> 5);
    if (__builtin_amdgcn_ballot_w64(mine)) {
      const int mt = tl >> 5, rt = (((tl & 31) >> 3) << 2) | (tl & 3);
      float t = 0.f;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (mi == mt && r == rt) t = acc[mi][ni][r];
      if (mine) a.tz[j] = t * a.c1;
    }
  }
}

// Loaders of the fused tiles: weight rows v0 .. (clamped below n_real) and the scored hidden
// rows j0 .. (clamped below the count), gathered through `scored` (ascending). The hidden
// resource starts at the tile's first scored row; the host keeps all T rows within 2^31 bytes
// (T * hidden_stride * 2 < 2^31), so every lane offset, plus the K step's scalar offset, stays
// below 2^31 and inside the resource's range.
template <int NW>
__device__ __forceinline__ void weight_hidden_loaders(const uint16_t* W, int64_t ldw, int64_t n_real,
                                                      int v0, const uint16_t* h, int64_t ldh,
                                                      const int32_t* scored, int j0, int Ts, int H,
                                                      dma::LoaderT<NW>& la, dma::LoaderT<NW>& lb) {
  const int nv = n_real - v0 < BM ? (int)(n_real - v0) : BM;
  const int nj = Ts - j0 < BN ? Ts - j0 : BN;
  // One address for the whole wave: readfirstlane keeps the resources in scalar registers also
  // where the compiler reads `scored` with vector loads (after stores it cannot prove
  // disjoint), which would otherwise put every DMA instruction in a per-lane loop.
  const int64_t h0 = __builtin_amdgcn_readfirstlane(scored[j0]);
  const int64_t hl = __builtin_amdgcn_readfirstlane(scored[j0 + nj - 1]);
  la.init(W + (int64_t)v0 * ldw, (uint64_t)((nv - 1) * ldw + H) * 2);
  lb.init(h + h0 * ldh, (uint64_t)((hl - h0) * ldh + H) * 2);
#pragma unroll
  for (int u = 0; u < dma::LoaderT<NW>::NIW; ++u) {
    const int r = dma::LoaderT<NW>::row_of(u);
    la.set(u, r < nv ? r : nv - 1, ldw);
    lb.set(u, scored[j0 + (r < nj ? r : nj - 1)] - h0, ldh);
  }
}

// The forward's LDS: the pipeline's two stages, then the epilogue's 6 x 256 fp32 partials and a
// word for tile claims. One array, not several: with a second LDS object the compiler can no
// longer tell the stages' DMA writes from the fragment reads and waits for every DMA load
// before each read.
constexpr int FWD_LDS_HALFS = dma::LDS_BYTES / 2 + 6 * 256 * 2 + 8;   // + the tile-claim slot
static_assert(dma::BKD == KSTEP, "K step shared with the host");
static_assert(QCTR_INTS > NUM_XCD, "queue counters and the all-empty flag");

// The forward tile runs FWD_WAVES = 8 waves, two per SIMD: each wave holds 128 x 64 outputs (128
// accumulators), so one wave's LDS reads, DMA issue and barrier waits overlap the other's
// MFMAs. Every output's MFMA chain and every token's reduction order are those of the 4-wave
// tile (1 wave per SIMD, 128 x 128 per wave). Kernels come one per bias mode, differing only in
// how the accumulators start: a run-time choice there makes the compiler spill accumulators in
// the epilogue.
constexpr int FWD_WAVES = 8;

template <int BMODE, int NFB>
__device__ __forceinline__ void fwd_init_acc(f32x16 (&acc)[4][NFB], const FwdArgs& a, int v0) {
  if constexpr (BMODE == BIAS_NONE) zero_acc(acc);
  else bias_acc<BMODE == BIAS_F32, NFB>(acc, a.bias, v0, a.n_real);
}

template <int NFB>
__device__ __forceinline__ void fwd_tile_epilogue(const f32x16 (&acc)[4][NFB], const FwdArgs& a,
                                                  int vt, int tb, int Ts, float* red) {
  const int v0 = vt * BM, j0 = tb * BN;
  if (v0 + BM > a.n_real) fwd_epilogue<true, NFB>(acc, a, vt, v0, j0, Ts, red);
  else fwd_epilogue<false, NFB>(acc, a, vt, v0, j0, Ts, red);
}

// The forward GEMM as persistent workers (the host launches one per compute unit, a multiple
// of NUM_XCD, when the K steps are even). XCD x owns a contiguous share of the logical tiles
// (its queue, as for the backward kernels). Worker wi of the XCD runs positions wi, wi + nwx,
// ... of the queue's static first three quarters, in the order one workgroup per tile would
// start them, then claims tiles of the dynamic last quarter one at a time (own XCD first, then
// the others'), so that workers of a faster XCD take over the tail of a slower one. Against
// one workgroup per tile this saves each tile's launch, address setup and first DMA round
// trip: the last two K steps of a tile load the first two of the worker's next tile, which
// land during the epilogue. Tiles past the scored rows are skipped. A tile's arithmetic is
// that of k_fwd_tiles, whoever runs it: results are bitwise the same.
template <int BMODE, int NW>
__global__ __launch_bounds__(64 * NW, 1) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void k_fwd(FwdArgs a) {
  constexpr int NFB = 16 / NW;
  __shared__ __attribute__((aligned(16))) uint16_t smem[FWD_LDS_HALFS];
  float* const red = reinterpret_cast<float*>(smem + dma::LDS_BYTES / 2);
  int* const slot = reinterpret_cast<int*>(red + 6 * 256);
  const int Ts = *a.count;
  const int ntiles = a.nvt * a.ntb;
  const int x = blockIdx.x % NUM_XCD, nwx = gridDim.x / NUM_XCD;
  const int qf = queue_first(ntiles, x), s0 = queue_static(queue_size(ntiles, x));
  int pos = blockIdx.x / NUM_XCD;   // the worker's next static position
  // The worker's next tile with scored rows: false when there is none.
  auto next_tile = [&](int& vt, int& tb) -> bool {
    for (;;) {
      int t;
      if (pos < s0) {
        t = qf + pos;
        pos += nwx;
      } else {
        if (threadIdx.x == 0) *slot = claim_dynamic(a.qctr, ntiles, x);
        dma::lds_barrier();
        t = *slot;
        dma::lds_barrier();   // every wave has read the slot before the next claim writes it
        if (t < 0) return false;
      }
      vocab_token_tile(t, a.nvt, a.ntb, vt, tb);
      if (tb * BN < Ts) return true;
    }
  };
  int vt = 0, tb = 0;
  if (!next_tile(vt, tb)) return;
  const int n = a.H / dma::BKD;
  dma::LoaderT<NW> la, lb, la2, lb2;
  weight_hidden_loaders<NW>(a.W, a.ldw, a.n_real, vt * BM, a.h, a.ldh, a.scored, tb * BN, Ts,
                            a.H, la, lb);
  bool primed = false;
  for (;;) {
    int vt2 = 0, tb2 = 0;
    const bool more = next_tile(vt2, tb2);
    if (more) {
      weight_hidden_loaders<NW>(a.W, a.ldw, a.n_real, vt2 * BM, a.h, a.ldh, a.scored, tb2 * BN,
                                Ts, a.H, la2, lb2);
    } else {
      la2 = la;
      lb2 = lb;
    }
    f32x16 acc[4][NFB];
    fwd_init_acc<BMODE, NFB>(acc, a, vt * BM);
    dma::mainloop_chain(la, lb, la2, lb2, primed, more, n, smem, acc);
    fwd_tile_epilogue<NFB>(acc, a, vt, tb, Ts, red);
    if (!more) break;
    vt = vt2;
    tb = tb2;
    la = la2;
    lb = lb2;
    primed = true;
  }
}

// One workgroup per tile in the static XCD order: the forward for an odd number of K steps,
// where the persistent workers' stage parity does not carry from one tile to the next.
template <int BMODE, int NW>
__global__ __launch_bounds__(64 * NW, 1) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void k_fwd_tiles(FwdArgs a) {
  constexpr int NFB = 16 / NW;
  __shared__ __attribute__((aligned(16))) uint16_t smem[FWD_LDS_HALFS];
  float* const red = reinterpret_cast<float*>(smem + dma::LDS_BYTES / 2);
  int vt, tb;
  vocab_token_tile(xcd_remap(blockIdx.x, gridDim.x), a.nvt, a.ntb, vt, tb);
  const int Ts = *a.count;
  if (tb * BN >= Ts) return;
  dma::LoaderT<NW> la, lb;
  weight_hidden_loaders<NW>(a.W, a.ldw, a.n_real, vt * BM, a.h, a.ldh, a.scored, tb * BN, Ts,
                            a.H, la, lb);
  f32x16 acc[4][NFB];
  fwd_init_acc<BMODE, NFB>(acc, a, vt * BM);
  dma::mainloop(la, lb, 0, a.H / dma::BKD, smem, acc);
  fwd_tile_epilogue<NFB>(acc, a, vt, tb, Ts, red);
}

// ------------------------------------------------------------------------------------
// Cross-tile combine, in vocabulary-tile order: chain c of 16 folds tiles c, c+16, ... of a row,
// then the row's 16 chains are folded in order c = 0..15. A workgroup takes 32 rows x 16 chains
// (thread = chain * 32 + row), so the 4096 rows of a chunk spread over 128 workgroups; the
// arithmetic of a row does not depend on that grouping. With d_k = m_k - M:
// S = sum_k s_k e^{d_k}, Q = sum_k e^{d_k}(q_k + s_k d_k log2 e); lse = M + ln S and
// entropy = ln S - ln2 * Q / S. An empty shard gives lse = -inf, entropy 0, target logit 0,
// in_range 0 and logp -inf ([top-p replay, "Changes" table]: empty vocabulary rows).
// ------------------------------------------------------------------------------------
__device__ __forceinline__ void fold(float& M, float& S, float& Q, float m, float s, float q) {
  // Combine (M, S, Q) with a partial (m, s, q); both may be empty (-inf max, zero sums).
  if (m == -INFINITY) return;
  if (M == -INFINITY) {
    M = m; S = s; Q = q;
    return;
  }
  const float N = fmaxf(M, m);
  const float da = M - N, db = m - N;
  const float wa = expf(da), wb = expf(db);
  Q = wa * (Q + S * da * kLog2e) + wb * (q + s * db * kLog2e);
  S = wa * S + wb * s;
  M = N;
}

// 32 rows: a wave's loads of one partial are 32 consecutive floats, a whole 128-byte line
// (with 16 rows two workgroups each fetched half of every line: 70 MB for 29 MB of partials).
constexpr int COMBINE_ROWS = 32, COMBINE_CHAINS = 16;

__global__ __launch_bounds__(COMBINE_ROWS * COMBINE_CHAINS) void k_combine(CombineArgs a) {
  __shared__ float rm[COMBINE_CHAINS][COMBINE_ROWS], rs[COMBINE_CHAINS][COMBINE_ROWS],
      rq[COMBINE_CHAINS][COMBINE_ROWS];
  const int r = threadIdx.x % COMBINE_ROWS, c = threadIdx.x / COMBINE_ROWS;
  const int Ts = *a.count;
  const int j = blockIdx.x * COMBINE_ROWS + r;
  if (blockIdx.x * COMBINE_ROWS >= Ts) return;
  float M = -INFINITY, S = 0.f, Q = 0.f;
  if (j < Ts) {
    // Unrolled so that each thread has several independent loads in flight.
    float mmax = -INFINITY;
#pragma unroll 8
    for (int vt = c; vt < a.nvt; vt += COMBINE_CHAINS)
      mmax = fmaxf(mmax, a.pm[(int64_t)vt * a.pstride + j]);
    if (mmax != -INFINITY) {
#pragma unroll 8
      for (int vt = c; vt < a.nvt; vt += COMBINE_CHAINS) {
        const int64_t o = (int64_t)vt * a.pstride + j;
        const float d = a.pm[o] - mmax, s = a.ps[o], q = a.pq[o];
        const float e = expf(d);
        S += e * s;
        Q += e * (q + s * d * kLog2e);
      }
      M = mmax;
    }
  }
  rm[c][r] = M;
  rs[c][r] = S;
  rq[c][r] = Q;
  __syncthreads();
  if (c != 0 || j >= Ts) return;
  M = -INFINITY; S = 0.f; Q = 0.f;
  for (int g = 0; g < COMBINE_CHAINS; ++g) fold(M, S, Q, rm[g][r], rs[g][r], rq[g][r]);
  float lse, ent;
  if (M == -INFINITY || !(S > 0.f)) {
    lse = -INFINITY;
    ent = 0.f;
  } else {
    const float ls = logf(S);
    lse = M + ls;
    ent = ls - kLn2 * (Q / S);
  }
  const int row = a.scored[j];
  const bool hit = a.tloc[j] >= 0;
  const float tz = hit ? a.tz[j] : 0.f;
  a.out_t[row] = tz;
  a.out_f[row] = hit ? 1 : 0;
  a.out_l[row] = lse;
  if (a.out_e) a.out_e[row] = ent;
  if (a.out_p) a.out_p[row] = hit ? tz - lse : -INFINITY;
}

// ------------------------------------------------------------------------------------
// Rank-ordered shard merge ([top-p replay, "Summary"]: rank-ordered reductions, shards with
// no candidates handled). One thread per row; shards r = 0..world-1 in order.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_merge(MergeArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= a.T) return;
  if (a.mask != nullptr && a.mask[t] == 0) {
    a.out_p[t] = 0.f;
    a.out_l[t] = 0.f;
    if (a.out_e) a.out_e[t] = 0.f;
    return;
  }
  float M = -INFINITY;
  for (int r = 0; r < a.world; ++r) M = fmaxf(M, a.lse[r][t]);
  float lse = -INFINITY;
  if (M != -INFINITY) {
    float S = 0.f;
    for (int r = 0; r < a.world; ++r) {
      const float L = a.lse[r][t];
      if (L != -INFINITY) S += expf(L - M);
    }
    lse = M + logf(S);
  }
  int found = -1;
  for (int r = 0; r < a.world && found < 0; ++r)
    if (a.flag[r][t]) found = r;
  if (found >= 0) {
    a.out_p[t] = a.tl[found][t] - lse;
  } else {
    a.out_p[t] = -INFINITY;
    if (a.status) atomicOr(a.status, LLP_STATUS_TARGET_NOT_FOUND);
  }
  a.out_l[t] = lse;
  if (a.out_e) {
    float ent = 0.f;
    if (lse != -INFINITY)
      for (int r = 0; r < a.world; ++r) {
        const float L = a.lse[r][t];
        if (L != -INFINITY) ent += expf(L - lse) * (a.ent[r][t] + (lse - L));
      }
    a.out_e[t] = ent;
  }
}

// ------------------------------------------------------------------------------------
// Compact top-p replay scorer ([top-p replay, "Summary"] and "Changes" table: validate the
// replay inputs, sort and deduplicate up to 64 ids, apply temperature, return local
// reductions; score the compact ids directly, no full-vocabulary keep mask). A wave64 per
// row (or per few rows): lane k holds slot k; ids inside the shard's real range become local keys, the rest a
// sentinel. The c keys are first packed into lanes 0..c-1 (in slot order), then a bitonic
// sort over the first P = 2^ceil(log2 c) lanes (the lanes past c hold the sentinel, the
// largest key, so they already sit in sorted position), adjacent dedup and compaction by
// ballot put the i-th distinct id on lane i: the fixed butterfly sum is independent of the
// order and multiplicity of the listed ids. A shard holds a handful of a nucleus's ids, so P
// is small and the sort takes a few stages instead of the 21 of a 64-lane network.
// ------------------------------------------------------------------------------------
// Scores a set of logits held one per lane in ascending-id order (lane i holds the i-th
// distinct id's z when `live`, else -inf): M = max, returns sum exp(z - M), both by a fixed
// butterfly, so the result is a function of the set alone. The compact and the dense
// keep-mask scorers both end here, which makes them bitwise equal on the same nucleus.
// `span` (a power of two in 1..64, wave-uniform) bounds the live lanes: they are all below
// it. The butterfly steps with off >= span only combine lane l < span with lanes whose values
// are -inf (max) and 0 (sum), which leaves lane l's value unchanged, so skipping them gives
// lanes below span, lane 0 included, the bits of the full 64-lane butterfly. Lanes at or
// past span return garbage; callers use lane 0.
__device__ __forceinline__ float wave_set_sum(float z, bool live, float& M, int span) {
  M = z;
  for (int off = span >> 1; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float e = live ? expf(z - M) : 0.f;
  for (int off = span >> 1; off > 0; off >>= 1) e += __shfl_xor(e, off);
  return e;
}

// Smallest power of two >= n (1 for n <= 1), n <= 64.
__device__ __forceinline__ int pow2_ceil(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

constexpr int TOPP_SENT = 0x7FFFFFFF;  // sorts after every local key

// One scored row by the whole wave: lane k holds slot k. The path of rows whose shard holds more
// than 16 of the row's listed ids; its bits are those of the grouped path below for any row
// both can score. zsw / ksw: this wave's 64-entry LDS scratch (private to the wave; one
// wave's LDS accesses complete in issue order).
__device__ __forceinline__ void topp_row64(const ToppArgs& a, int64_t row, int lane, float* zsw,
                                           int* ksw) {
  int64_t id = lane < a.K ? a.ids[row * a.ids_stride + lane] : -1;
  if (id < -1 || id >= a.real_vocab) id = -1;   // its status bit is set by the grouped pass
  const int64_t loc = id - a.offset;
  const bool in_shard = id >= 0 && loc >= 0 && loc < a.n_real;
  const uint64_t vb = __builtin_amdgcn_ballot_w64(in_shard);
  const int c = __popcll(vb);
  if (in_shard)
    ksw[__builtin_amdgcn_mbcnt_hi((uint32_t)(vb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)vb, 0))] =
        (int)loc;
  __builtin_amdgcn_wave_barrier();
  int key = lane < c ? ksw[lane] : TOPP_SENT;
  const int P = pow2_ceil(c);
  for (int k = 2; k <= P; k <<= 1)
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      const int other = __shfl_xor(key, jj);
      const bool up = (lane & k) == 0, lower = (lane & jj) == 0;
      key = (lower == up) ? min(key, other) : max(key, other);
    }
  const int prev = __shfl_up(key, 1);
  const bool keep = key != TOPP_SENT && (lane == 0 || key != prev);
  const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
  const int n = __popcll(bal);
  const int64_t tg = a.targets[row];
  const uint64_t tb = __builtin_amdgcn_ballot_w64(keep && (int64_t)key == tg - a.offset);
  if (keep) {
    const int64_t o = row * a.lstride + key;
    const float x = a.bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(a.logits)[o])
                           : reinterpret_cast<const float*>(a.logits)[o];
    zsw[__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0))] =
        x * a.c1;
  }
  __builtin_amdgcn_wave_barrier();
  float M;
  const float e = wave_set_sum(lane < n ? zsw[lane] : -INFINITY, lane < n, M, pow2_ceil(n));
  if (lane == 0) {
    const float lse = M + logf(e);   // n >= 1: the shard holds more than 16 listed ids
    const float t = tb ? zsw[__popcll(bal & ((tb & (0 - tb)) - 1))] : 0.f;
    a.out_t[row] = t;
    a.out_f[row] = tb ? 1 : 0;
    a.out_l[row] = lse;
    if (a.out_p) a.out_p[row] = tb ? t - lse : -INFINITY;
  }
}

// A wave scores 4 consecutive rows at once, 16 lanes per row (group g = lane / 16 takes row
// row0 + g, lane l of the group slots l, l + 16, l + 32, l + 48). A group packs its row's
// in-shard keys into its lanes (at most 16; a row with more goes to topp_row64 afterwards),
// sorts them with the bitonic network over the wave-wide largest power of two P <= 16 that
// any group needs (partners l ^ jj, jj < P, stay in the group; extra stages leave a sorted
// group unchanged), dedups, compacts, gathers and sums with wave_set_sum, whose steps off < 16
// stay in the group: lane 16g pairs with the group's lanes exactly as lane 0 pairs with lanes
// 0..15 in the whole-wave form, and every other partner adds a zero (or -inf to the max), so
// each row gets the bits of the whole-wave path.
__global__ __launch_bounds__(256) void k_topp(ToppArgs a) {
  __shared__ float zs[4][64];
  __shared__ int ks[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, gl = lane & 15;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + w) * 4;
  if (row0 >= a.T) return;
  const int64_t row = row0 + g;
  const bool in_rows = row < a.T;
  const int64_t rr = in_rows ? row : a.T - 1;   // a group past T reads the last row, writes nothing
  const bool scored = in_rows && (a.mask == nullptr || a.mask[rr] != 0);
  const int64_t tg = a.targets[rr];
  int status = 0;
  int64_t id[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int sl = gl + 16 * j;
    id[j] = sl < a.K ? a.ids[rr * a.ids_stride + sl] : -1;
  }
  const uint64_t gm = 0xFFFFull << (16 * g);
  const uint64_t lower = (1ull << lane) - 1;
  int c = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int64_t v = id[j];
    if (v < -1 || v >= a.real_vocab) {
      if (in_rows) status |= LLP_STATUS_REPLAY_ID_INVALID;
      v = -1;
    }
    const int64_t loc = v - a.offset;
    const bool ins = scored && v >= 0 && loc >= 0 && loc < a.n_real;
    const uint64_t bj = __builtin_amdgcn_ballot_w64(ins) & gm;
    const int pos = c + __popcll(bj & lower);
    if (ins && pos < 16) ks[w][16 * g + pos] = (int)loc;
    c += __popcll(bj);
  }
  const bool wide = c > 16;
  __builtin_amdgcn_wave_barrier();
  int key = (!wide && gl < c) ? ks[w][16 * g + gl] : TOPP_SENT;
  int P = pow2_ceil(wide ? 1 : c);
  P = max(P, __shfl_xor(P, 16));
  P = max(P, __shfl_xor(P, 32));
  P = __builtin_amdgcn_readfirstlane(P);
  for (int k = 2; k <= P; k <<= 1)
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      // Direction from the lane's index in its group: at k = 16 every group sorts ascending.
      const int other = __shfl_xor(key, jj);
      const bool up = (gl & k) == 0, lo = (gl & jj) == 0;
      key = (lo == up) ? min(key, other) : max(key, other);
    }
  const int prev = __shfl_up(key, 1);
  const bool keep = key != TOPP_SENT && (gl == 0 || key != prev);
  const uint32_t gb = (uint32_t)((__builtin_amdgcn_ballot_w64(keep) & gm) >> (16 * g));
  const uint32_t tbg =
      (uint32_t)((__builtin_amdgcn_ballot_w64(keep && (int64_t)key == tg - a.offset) & gm) >> (16 * g));
  const int n = __popc(gb);
  if (keep) {
    const int64_t o = row * a.lstride + key;
    const float x = a.bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(a.logits)[o])
                           : reinterpret_cast<const float*>(a.logits)[o];
    zs[w][16 * g + __popc(gb & ((1u << gl) - 1))] = x * a.c1;
  }
  __builtin_amdgcn_wave_barrier();
  int span = pow2_ceil(n);
  span = max(span, __shfl_xor(span, 16));
  span = max(span, __shfl_xor(span, 32));
  span = __builtin_amdgcn_readfirstlane(span);
  float M;
  const float e = wave_set_sum(gl < n ? zs[w][16 * g + gl] : -INFINITY, gl < n, M, span);
  if (scored && (tg < 0 || tg >= a.real_vocab)) status |= LLP_STATUS_TARGET_OUT_OF_RANGE;
  if (gl == 0 && in_rows && !wide) {
    if (!scored) {
      a.out_t[row] = 0.f;
      a.out_f[row] = 0;
      a.out_l[row] = 0.f;
      if (a.out_p) a.out_p[row] = 0.f;
    } else if (n == 0) {
      a.out_t[row] = 0.f;
      a.out_f[row] = 0;
      a.out_l[row] = -INFINITY;
      if (a.out_p) a.out_p[row] = -INFINITY;
    } else {
      const float lse = M + logf(e);
      // The target's compact position = kept lanes of the group below the one holding it.
      const float t = tbg ? zs[w][16 * g + __popc(gb & ((tbg & (0u - tbg)) - 1))] : 0.f;
      a.out_t[row] = t;
      a.out_f[row] = tbg ? 1 : 0;
      a.out_l[row] = lse;
      if (a.out_p) a.out_p[row] = tbg ? t - lse : -INFINITY;
    }
  }
  // Rows whose shard holds more than 16 of their ids: the whole wave, one row at a time.
  uint64_t wb = __builtin_amdgcn_ballot_w64(wide && gl == 0);
  while (wb) {
    const int gg = __builtin_ctzll(wb) >> 4;
    wb &= wb - 1;
    topp_row64(a, row0 + gg, lane, zs[w], ks[w]);
  }
  if (a.status) {
    const uint64_t any = __builtin_amdgcn_ballot_w64(status != 0);
    if (any) {
      int st = status;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) st |= __shfl_xor(st, off);
      if (lane == 0) atomicOr(a.status, st);
    }
  }
}

// ------------------------------------------------------------------------------------
// Backward. G[j, v] = (dlogp (1[v = target] - p) - dentropy p (z - E_p z)) / tau with
// p = exp(z - lse) is recomputed tile by tile with the forward's tile, rounded to bf16 and
// written as G[scored row j][local column v] (zeros in excluded columns). Then
// dhidden = G W (split over K = vocabulary in a fixed number of fixed ranges, partials
// summed in range order) and dweight += G^T h over the scored rows in order, db += sum_j G.
// ------------------------------------------------------------------------------------
constexpr int GT_STRIDE = BN + 8;  // padded LDS row (bf16 elements) of the staged G tile
constexpr int GRAD_LDS_BYTES = BN * GT_STRIDE * 2;
static_assert(GRAD_LDS_BYTES <= 160 * 1024, "gradient tile LDS");
constexpr int BWDG_LDS_BYTES = GRAD_LDS_BYTES > dma::LDS_BYTES ? GRAD_LDS_BYTES : dma::LDS_BYTES;

// Writes the staged bf16 tile Gs[token][vocab] (LDS) as G rows, including the zero rows from
// the count up to the next whole K step (the dweight product reads G K-major in steps of 64).
// Non-temporal stores: G (1.24 GB at T = 4096) is far larger than the caches, so its lines
// would be gone before the next kernels read them; cached, they would evict operand lines
// that other tiles re-read (the stores as NT measured ~0.6% off the backward).
template <int NTHR>
__device__ __forceinline__ void grad_store(const GradArgs& a, int v0, int j0, int Ts,
                                           const uint16_t* smem) {
  const int tpad = (Ts + KSTEP - 1) / KSTEP * KSTEP;
  __syncthreads();
  for (int idx = threadIdx.x; idx < BN * (BM / 8); idx += NTHR) {
    const int tn = idx >> 5, c = idx & 31;
    const int j = j0 + tn;
    if (j < tpad)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(smem + tn * GT_STRIDE + c * 8),
                                  reinterpret_cast<u32x4*>(a.G + (int64_t)j * a.ldg + v0 + c * 8));
  }
}

// NFB = 4: 4 waves of 128 vocabulary x 128 tokens (accumulators in AGPRs, read with acc_read);
// NFB = 2: 8 waves of 128 x 64 (accumulators in VGPRs). G's values do not depend on the layout.
template <bool TAIL, bool ENT, int NFB>
__device__ __forceinline__ void grad_epilogue(f32x16 (&acc)[4][NFB], const GradArgs& a, int v0,
                                              int j0, int Ts, uint16_t* smem) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  constexpr int TW = 32 * NFB;  // tokens per wave
  const int vbase = v0 + wm * 128;
  const float c1l = a.c1 * kLog2e;
  // Per row: dlc = dlogp / tau and dec = dentropy / tau, both 0 for rows past the count and rows
  // no gradient flows into, so those rows come out as exact (+0) zeros in G.
  float lsel[NFB], dlc[NFB], dec[NFB], ez[NFB];
  int tl[NFB];
#pragma unroll
  for (int ni = 0; ni < NFB; ++ni) {
    const int j = j0 + wn * TW + ni * 32 + (lane & 31);
    const int jj = j < Ts ? j : Ts - 1;
    const int row = a.scored[jj];
    const float lse = a.lse[row];
    lsel[ni] = lse * kLog2e;
    const float dl = a.dlogp[row];
    const float de = ENT ? a.dent[row] : 0.f;
    const bool live = j < Ts && (dl != 0.f || de != 0.f);
    dlc[ni] = live ? dl * a.c1 : 0.f;
    dec[ni] = live ? de * a.c1 : 0.f;
    ez[ni] = ENT ? lse - a.ent[row] : 0.f;
    tl[ni] = a.tloc[jj] - a.toff - vbase;
  }
  // Stage the bf16 tile as Gs[token][vocab] in LDS, then write full rows.
  __syncthreads();
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int ni = 0; ni < NFB; ++ni) {
      const int tn = wn * TW + ni * 32 + (lane & 31);
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        float gv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = rg * 4 + u;
          const int vl = mi * 32 + mfma_row(r, lane);
          const float x = NFB == 4 ? acc_read(acc[mi][ni][r]) : acc[mi][ni][r];
          // p = exp(z - lse) = 2^(x c1 log2(e) - lse log2(e));
          // g = (dlogp (1[v = t] - p) - dentropy p (z - E z)) / tau.
          const float p = __builtin_amdgcn_exp2f(fmaf(x, c1l, -lsel[ni]));
          float g = fmaf(-dlc[ni], p, vl == tl[ni] ? dlc[ni] : 0.f);
          if constexpr (ENT) g = fmaf(-dec[ni] * p, fmaf(x, a.c1, -ez[ni]), g);
          if (TAIL && vbase + vl >= a.n_real) g = 0.f;
          gv[u] = g;
        }
        const uint32_t pk[2] = {pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3])};
        const int vl0 = wm * 128 + mi * 32 + mfma_row(rg * 4, lane);
        *reinterpret_cast<uint2*>(smem + tn * GT_STRIDE + vl0) = make_uint2(pk[0], pk[1]);
      }
    }
  }
  grad_store<16 * 64 / NFB>(a, v0, j0, Ts, smem);
}

// Waves of the gradient tile (4: one per SIMD, 128 x 128 each; 8: two per SIMD, 128 x 64). Both
// give the same G; 8 waves measured 2.3% slower here (4.22 against 4.13 ms at T=4096), unlike
// the forward, whose epilogue stages nothing through LDS.
constexpr int GRAD_WAVES = 4;

template <int NW>
__global__ __launch_bounds__(64 * NW, 1) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void k_grad(GradArgs a) {
  constexpr int NFB = 16 / NW;
  __shared__ __attribute__((aligned(16))) uint16_t smem[BWDG_LDS_BYTES / 2];
  const int tile = take_tile(a.qctr, a.nvt * a.ntb, reinterpret_cast<int*>(smem));
  if (tile < 0) return;
  int vt, tb;
  vocab_token_tile(tile, a.nvt, a.ntb, vt, tb);
  const int Ts = *a.count;
  const int j0 = tb * BN, v0 = vt * BM;
  if (j0 >= Ts) return;
  dma::LoaderT<NW> la, lb;
  weight_hidden_loaders<NW>(a.W, a.ldw, a.n_real, v0, a.h, a.ldh, a.scored, j0, Ts, a.H, la, lb);
  f32x16 acc[4][NFB];
  init_acc(acc, a.bias, a.bias_f32, v0, a.n_real);
  dma::mainloop(la, lb, 0, a.H / dma::BKD, smem, acc);
  const bool tail = v0 + BM > a.n_real;
  if (a.dent != nullptr) {
    if (tail) grad_epilogue<true, true, NFB>(acc, a, v0, j0, Ts, smem);
    else grad_epilogue<false, true, NFB>(acc, a, v0, j0, Ts, smem);
  } else {
    if (tail) grad_epilogue<true, false, NFB>(acc, a, v0, j0, Ts, smem);
    else grad_epilogue<false, false, NFB>(acc, a, v0, j0, Ts, smem);
  }
  // Bias gradient: this tile's column sums of the bf16 G it wrote (still staged in LDS as
  // Gs[token][vocab]), rows in order; rows past the count are zero.
  if (a.dbp != nullptr) {
    for (int c = threadIdx.x; c < BM; c += 64 * NW) {
      float sum = 0.f;
      for (int tn = 0; tn < BN; ++tn) sum += bf16_to_f32(smem[tn * GT_STRIDE + c]);
      a.dbp[(int64_t)tb * a.ldg + v0 + c] = sum;
    }
  }
}

// dhidden partials: P[split][j][n] = sum over the split's K range of G[j, k] W[k, n]
// (K = local vocabulary column; G is zero past the real columns, and weight rows past the
// last real one are read as that row). With G held one vocabulary slab at a time, each slab
// after the first adds its product into P (slabs in order, so the sum's order is fixed).
// Tiles: grouped like the vocabulary x token grids with M = scored-row tiles.
// Waves of the dhidden tile (4: one per SIMD, 128 x 128 each; 8: two per SIMD, 128 x 64). Both
// give the same partials; 8 waves measured 3.6% slower here (4.09 against 3.94 ms at T=4096).
constexpr int DH_WAVES = 4;

template <int NW, bool ACC>
__device__ __forceinline__ void dh_tile(const DhArgs& a) {
  constexpr int NFB = 16 / NW;
  __shared__ __attribute__((aligned(16))) uint16_t smem[dma::LDS_BYTES / 2];
  const int per = a.ntm * a.ntn;
  const int tile = take_tile(a.qctr, per * a.nsplit, reinterpret_cast<int*>(smem));
  if (tile < 0) return;
  const int sp = tile / per;
  int mt, nt;
  vocab_token_tile(tile % per, a.ntm, a.ntn, mt, nt);
  const int Ts = *a.count;
  const int j0 = mt * BM, n0 = nt * BN;
  if (j0 >= Ts) return;
  // A: G rows j0 .. j0+255 (inside the workspace's row capacity), K = local vocabulary.
  // B: the weight itself, K-major: rows = vocabulary (up to the last real one), columns
  // n0 .. (< H).
  const int nn = a.H - n0 < BN ? a.H - n0 : BN;
  const int64_t kb = (int64_t)a.nks * dma::BKD;
  dma::LoaderT<NW> la;
  la.init(a.G + (int64_t)j0 * a.ldg, (uint64_t)((BM - 1) * a.ldg + kb) * 2);
#pragma unroll
  for (int u = 0; u < dma::LoaderT<NW>::NIW; ++u) la.set(u, dma::LoaderT<NW>::row_of(u), a.ldg);
  dma::LoaderKT<NW> lb;
  lb.init(a.W + n0, a.ldw, (int)a.n_real - 1, nn);
  const int ks0 = (int)((int64_t)a.nks * sp / a.nsplit);
  const int ks1 = (int)((int64_t)a.nks * (sp + 1) / a.nsplit);
  f32x16 acc[4][NFB];
  zero_acc(acc);
  dma::mainloop(la, lb, ks0, ks1, smem, acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave & 1, wn = wave >> 1;
  float* P = a.P + (int64_t)sp * a.pstride * a.H;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < NFB; ++ni) {
      const int n = n0 + wn * 32 * NFB + ni * 32 + (lane & 31);
      float old[16];
      if constexpr (ACC) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + wm * 128 + mi * 32 + mfma_row(r, lane);
          old[r] = j < Ts && n < a.H ? P[(int64_t)j * a.H + n] : 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + wm * 128 + mi * 32 + mfma_row(r, lane);
        if (j < Ts && n < a.H) P[(int64_t)j * a.H + n] = ACC ? old[r] + acc[mi][ni][r] : acc[mi][ni][r];
      }
      // One 16-value block at a time: the old values of later blocks are not loaded early.
      if constexpr (ACC) __builtin_amdgcn_sched_barrier(0);
    }
}

// dhidden[row] = bf16(sum over splits in order); unscored rows are zero.
// The dhidden product (first vocabulary slab, or the only one) and the same product added into
// the partials of the slabs before it.
template <int NW>
__global__ __launch_bounds__(64 * NW, 1) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void k_dh(DhArgs a) {
  dh_tile<NW, false>(a);
}
template <int NW>
__global__ __launch_bounds__(64 * NW, 1) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void k_dh_acc(DhArgs a) {
  dh_tile<NW, true>(a);
}

__global__ __launch_bounds__(256) void k_dh_reduce(DhReduceArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t cpr = a.H / 8;  // 8-column chunks per row
  if (idx >= a.T * cpr) return;
  const int64_t t = idx / cpr;
  const int n = (int)(idx % cpr) * 8;
  const int j = a.pos[t];
  uint32_t pk[4] = {0u, 0u, 0u, 0u};
  if (j >= 0) {
    float s[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) s[u] = 0.f;
    for (int sp = 0; sp < a.nsplit; ++sp) {
      const float* P = a.P + ((int64_t)sp * a.pstride + j) * a.H + n;
#pragma unroll
      for (int u = 0; u < 8; ++u) s[u] += P[u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      pk[u] = pack_bf16x2(s[2 * u], s[2 * u + 1]);
  }
  *reinterpret_cast<u32x4*>(a.dH + t * a.ldd + n) = u32x4{pk[0], pk[1], pk[2], pk[3]};
}

// dweight += the tile. The tile's rows are vocabulary rows (M: A = G read K-major) and its
// columns hidden columns (N: B = hgT, K contiguous), so lane l of block (mi, ni) holds hidden
// column n = wn*128 + ni*32 + (l & 31) of rows m = wm*128 + mi*32 + mfma_row(r, l): one store
// instruction (fixed mi, ni, r) writes 2 rows x 32 consecutive fp32 columns, two whole
// 128-byte lines. Stores and the old values' loads go through a buffer resource over the
// tile's real rows: rows at or past n_real are out of its range, and lanes whose column is at
// or past H get an offset past the range, so the hardware drops those stores (and reads 0).
// The dweight traffic is non-temporal (cache policy NT): it is touched once per call.
struct DwOut {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t vb[4];    // per block column ni: this lane's byte offset of (row wm*128 + 4(l >> 5),
                     // column wn*128 + ni*32 + (l & 31)), or DW_OUT_OF_RANGE past column H
  uint32_t rstride;  // bytes per dweight row
};
constexpr uint32_t DW_OUT_OF_RANGE = 0x80000000u;
constexpr int DW_CPOL = 2;  // buffer instruction cache policy: NT

__device__ __forceinline__ DwOut dw_out(const DwArgs& a, int m0, int n0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave & 1, wn = wave >> 1;
  const int nv = a.n_real - m0 < BM ? (int)(a.n_real - m0) : BM;
  const int nc = a.H - n0 < BN ? a.H - n0 : BN;
  DwOut o;
  o.rstride = (uint32_t)(a.lddw * 4);
  o.rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(a.dW + (int64_t)m0 * a.lddw + n0), (short)0,
                                             (int)((uint32_t)nv * o.rstride), 0x00020000);
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    const int col = wn * 128 + ni * 32 + (lane & 31);
    o.vb[ni] = col < nc ? (uint32_t)(wm * 128 + 4 * (lane >> 5)) * o.rstride + (uint32_t)col * 4u
                        : DW_OUT_OF_RANGE;
  }
  return o;
}

// Byte offset of accumulator (mi, ni, r) of this lane (past the range when masked: the row
// term is below 2^31 and DW_OUT_OF_RANGE is 2^31, so the sum does not wrap).
__device__ __forceinline__ uint32_t dw_off(const DwOut& o, int mi, int ni, int r) {
  return o.vb[ni] + (uint32_t)(mi * 32 + 8 * (r >> 2) + (r & 3)) * o.rstride;
}

// dweight[v, n] += sum_j G[j, v] hgT[n, j] over the scored rows j in ascending order
// (G and hgT are zero from the count up to the next whole K step). OVERWRITE: dweight[v, n] =
// that sum instead, written as +0 when no row is scored (a sum that starts at +0 is never -0,
// so this is bitwise the accumulate form applied to a zeroed dweight).
template <bool OVERWRITE>
__global__ __launch_bounds__(NTHREADS, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_dw(DwArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[dma::LDS_BYTES / 2];
  const int tile = take_tile(a.qctr, a.ntm * a.ntn, reinterpret_cast<int*>(smem));
  if (tile < 0) return;
  const int Ts = *a.count;
  if (!OVERWRITE && Ts <= 0) return;
  int mt, nt;
  vocab_token_tile<4>(tile, a.ntm, a.ntn, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  f32x16 acc[4][4];
  zero_acc(acc);
  if (Ts > 0) {
    // A (tile rows): G itself, K-major: rows = scored rows (zero from the count to the next
    // whole step), columns m0 .. m0+255 (inside the padded vocabulary capacity).
    // B (tile columns): hgT rows n0 .. (< H), K = scored rows rounded up to whole steps.
    const int nn = a.H - n0 < BN ? a.H - n0 : BN;
    const int nk = (Ts + dma::BKD - 1) / dma::BKD;
    const int64_t kb = (int64_t)nk * dma::BKD;
    dma::LoaderK la;
    la.init(a.G + m0, a.ldg, (int)kb - 1, BM);
    dma::Loader lb;
    lb.init(a.hgT + (int64_t)n0 * a.ldk, (uint64_t)((nn - 1) * a.ldk + kb) * 2);
#pragma unroll
    for (int u = 0; u < dma::NI; ++u) {
      const int r = dma::Loader::row_of(u);
      lb.set(u, r < nn ? r : nn - 1, a.ldk);
    }
    dma::mainloop(la, lb, 0, nk, smem, acc);
  }
  const DwOut o = dw_out(a, m0, n0);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    if constexpr (OVERWRITE) {
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __builtin_amdgcn_raw_buffer_store_b32(
              __builtin_bit_cast(uint32_t, acc_read(acc[mi][ni][r])), o.rsrc,
              (int)dw_off(o, mi, ni, r), 0, DW_CPOL);
    } else {
      // The block row's 64 old values, then their sums.
      uint32_t old[4][16];
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          old[ni][r] = __builtin_amdgcn_raw_buffer_load_b32(o.rsrc, (int)dw_off(o, mi, ni, r), 0,
                                                            DW_CPOL);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __builtin_amdgcn_raw_buffer_store_b32(
              __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, old[ni][r]) +
                                               acc_read(acc[mi][ni][r])),
              o.rsrc, (int)dw_off(o, mi, ni, r), 0, DW_CPOL);
    }
  }
}

// p[r * ld + c] = 0 for rows r0 <= r < r1 and columns c < cols (grid-stride, one float per
// thread and pass): padding rows of dweight/dbias, or all of them for a call with no rows, in
// overwrite mode.
__global__ __launch_bounds__(256) void k_zero_rows(ZeroArgs a) {
  const int64_t n = (a.r1 - a.r0) * a.cols;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    a.p[(a.r0 + i / a.cols) * a.ld + i % a.cols] = 0.f;
}

// out[c][r] = in[row(r)][c] for r < nvalid (zero for nvalid <= r < the grid's rows), 64 x 64
// bf16 tiles through LDS. row(r) = idx[r] when an index list is given, else r; nvalid is
// *count when given. Makes hgT (gathered hidden rows, transposed).
__global__ __launch_bounds__(256) void k_transpose(TransposeArgs a) {
  __shared__ uint16_t t[64][66];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int nvalid = a.count ? *a.count : (int)a.nvalid;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int r = q >> 3, cc = q & 7;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r0 + r < nvalid) {
      const int64_t row = a.idx ? a.idx[r0 + r] : r0 + r;
      v = *reinterpret_cast<const u32x4*>(a.in + row * a.ldi + c0 + cc * 8);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      t[r][cc * 8 + 2 * e] = (uint16_t)(v[e] & 0xFFFFu);
      t[r][cc * 8 + 2 * e + 1] = (uint16_t)(v[e] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int c = q >> 3, rc = q & 7;
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = (uint32_t)t[rc * 8 + 2 * e][c] | ((uint32_t)t[rc * 8 + 2 * e + 1][c] << 16);
    *reinterpret_cast<u32x4*>(a.out + (int64_t)(c0 + c) * a.ldo + r0 + rc * 8) = o;
  }
}

// dbias[v] (+)= sum over the token blocks tb = 0, 1, ... (in order) of the gradient tiles'
// column sums dbp[tb][v] (each the sum of the tile's 256 bf16 G values of column v, rows in
// order). Only the token blocks holding scored rows ran; G is zero past the count.
__global__ __launch_bounds__(256) void k_dbias(DbArgs a) {
  const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (v >= a.n_real) return;
  const int nb = (*a.count + BN - 1) / BN;
  float s = 0.f;
  for (int tb = 0; tb < nb; ++tb) s += a.dbp[(int64_t)tb * a.ldp + v];
  a.db[v] = a.overwrite ? s : a.db[v] + s;
}

// ------------------------------------------------------------------------------------
// Launchers (host). Each returns the launch status.
// ------------------------------------------------------------------------------------
static inline int ceil_div64(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// ------------------------------------------------------------------------------------
// Logits-input forward ([CUDA provider, "Megatron integration"]: reuse the LM head's local
// logits, no second projection). One workgroup per row streams the row's real columns once:
// each thread keeps a running (m, s, q) with s = sum 2^d, q = sum 2^d d, d = (z - m) log2 e,
// z = x * fl32(1/tau), over 8 columns at a time (rescaled when a chunk raises m); the 256
// partials are folded in a fixed order (lanes by halving strides, then waves 0..3) with the
// tile combine's algebra. Outputs and status bits as llp_forward's.
// ------------------------------------------------------------------------------------
__device__ __forceinline__ void load8(const void* base, int bf16, int64_t o, float (&x)[8]) {
  if (bf16) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + o);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __builtin_bit_cast(float, v[k] << 16);
      x[2 * k + 1] = __builtin_bit_cast(float, v[k] & 0xFFFF0000u);
    }
  } else {
    const float4 u = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + o);
    const float4 v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + o + 4);
    x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
    x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
  }
}

__device__ __forceinline__ float load1(const void* base, int bf16, int64_t o) {
  return bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[o])
              : reinterpret_cast<const float*>(base)[o];
}

// Adds z values (already scaled) to a running (m, s, q); zmax is their maximum.
template <int N>
__device__ __forceinline__ void online_add(float& m, float& s, float& q, const float (&z)[N],
                                           float zmax) {
  if (zmax > m) {
    if (m != -INFINITY) {
      const float dl = (m - zmax) * kLog2e;  // < 0
      const float f = __builtin_amdgcn_exp2f(dl);
      q = f * fmaf(dl, s, q);
      s = f * s;
    }
    m = zmax;
  }
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const float d = (z[k] - m) * kLog2e;
    const float e = __builtin_amdgcn_exp2f(d);
    s += e;
    q = fmaf(e, d, q);
  }
}

__global__ __launch_bounds__(256) void k_logits(LogitsArgs a) {
  __shared__ float pm[4], ps[4], pq[4];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int status = 0;
  if (row == 0 && a.cu_seqlens != nullptr) {
    for (int i = tid; i <= a.num_seqs; i += 256) {
      const int c = a.cu_seqlens[i];
      if (i == 0 && c != 0) status |= LLP_STATUS_LAYOUT_INVALID;
      if (i == a.num_seqs && (int64_t)c != a.T) status |= LLP_STATUS_LAYOUT_INVALID;
      if (i < a.num_seqs && a.cu_seqlens[i + 1] < c) status |= LLP_STATUS_LAYOUT_INVALID;
    }
    if (status && a.status) atomicOr(a.status, status);
    status = 0;
  }
  if (a.mask != nullptr && a.mask[row] == 0) {
    if (tid == 0) {
      a.out_t[row] = 0.f;
      a.out_f[row] = 0;
      a.out_l[row] = 0.f;
      if (a.out_e) a.out_e[row] = 0.f;
      if (a.out_p) a.out_p[row] = 0.f;
    }
    return;
  }
  const void* xr = a.bf16 ? (const void*)(reinterpret_cast<const uint16_t*>(a.logits) + row * a.ld)
                          : (const void*)(reinterpret_cast<const float*>(a.logits) + row * a.ld);
  const int64_t n = a.n_real, n8 = n & ~(int64_t)7;
  float m = -INFINITY, s = 0.f, q = 0.f;
  for (int64_t c = 8 * (int64_t)tid; c < n8; c += 8 * 256) {
    float x[8];
    load8(xr, a.bf16, c, x);
    float xm = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                     fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    float z[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) z[k] = x[k] * a.c1;
    online_add<8>(m, s, q, z, xm * a.c1);  // c1 > 0: the scaled max is the max of z
  }
  if (n8 + tid < n) {
    const float z[1] = {load1(xr, a.bf16, n8 + tid) * a.c1};
    online_add<1>(m, s, q, z, z[0]);
  }
  // Fold lanes in a fixed order: lane i takes lane i + off for off = 32, 16, ..., 1.
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float om = __shfl_down(m, off), os = __shfl_down(s, off), oq = __shfl_down(q, off);
    if (lane < off) fold(m, s, q, om, os, oq);
  }
  if (lane == 0) {
    pm[w] = m;
    ps[w] = s;
    pq[w] = q;
  }
  __syncthreads();
  if (tid != 0) return;
  float M = -INFINITY, S = 0.f, Q = 0.f;
  for (int g = 0; g < 4; ++g) fold(M, S, Q, pm[g], ps[g], pq[g]);
  float lse, ent;
  if (M == -INFINITY || !(S > 0.f)) {
    lse = -INFINITY;
    ent = 0.f;
  } else {
    const float ls = logf(S);
    lse = M + ls;
    ent = ls - kLn2 * (Q / S);
  }
  const int64_t tg = a.targets[row];
  const bool valid = tg >= 0 && tg < a.real_vocab;
  const int64_t loc = tg - a.offset;
  const bool hit = valid && loc >= 0 && loc < n;
  if (!valid) status |= LLP_STATUS_TARGET_OUT_OF_RANGE;
  if (!hit && a.world == 1) status |= LLP_STATUS_TARGET_NOT_FOUND;
  const float t = hit ? load1(xr, a.bf16, loc) * a.c1 : 0.f;
  a.out_t[row] = t;
  a.out_f[row] = hit ? 1 : 0;
  a.out_l[row] = lse;
  if (a.out_e) a.out_e[row] = ent;
  if (a.out_p) a.out_p[row] = hit ? t - lse : -INFINITY;
  if (status && a.status) atomicOr(a.status, status);
}

// ------------------------------------------------------------------------------------
// Dense keep-mask replay ([top-p replay, "Changes" table]: local logits reused with a keep
// mask, excluded entries -inf; [top-p replay, "Validation"]: bitwise equal to the compact
// scorer across shard offsets and empty shards). One wave per row scans the mask row in
// ascending column order (16 bytes per lane per step, an exclusive scan of the kept counts
// gives each kept column its rank; steps without a kept column skip the scan). The mask is
// read once per call, with non-temporal loads (11% faster than cached ones here). With at most 64 kept columns the i-th goes to lane i and
// the row is scored by wave_set_sum exactly as the compact scorer scores its sorted ids;
// larger sets (which the compact form cannot hold) are scored from per-lane running sums
// kept during the scan, folded by a fixed butterfly.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_keep(KeepArgs a) {
  __shared__ int list[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + w;
  if (row >= a.T) return;
  int status = 0;
  if (a.mask != nullptr && a.mask[row] == 0) {
    if (lane == 0) {
      a.out_t[row] = 0.f;
      a.out_f[row] = 0;
      a.out_l[row] = 0.f;
      if (a.out_p) a.out_p[row] = 0.f;
    }
    return;
  }
  const uint8_t* kr = a.keep + row * a.kstride;
  const void* xr = a.bf16 ? (const void*)(reinterpret_cast<const uint16_t*>(a.logits) + row * a.lstride)
                          : (const void*)(reinterpret_cast<const float*>(a.logits) + row * a.lstride);
  const int64_t n = a.n_real;
  int total = 0;                      // kept columns so far (wave-uniform)
  float lm = -INFINITY, ls = 0.f;     // this lane's running max and sum of exp (large sets)
  for (int64_t c4 = 0; c4 < n; c4 += 4096) {
    // Four 1 KiB pieces per pass, loaded together (independent loads in flight), then
    // scanned in column order.
    u32x4 v4[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int64_t cl = c4 + 1024 * p + 16 * lane;
      v4[p] = cl < n ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kr + cl))
                     : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int64_t cl = c4 + 1024 * p + 16 * lane;
      if (c4 + 1024 * p >= n) break;
      uint32_t bits = 0;
      if (cl < n) {
        const u32x4 v = v4[p];
#pragma unroll
        for (int k = 0; k < 16; ++k)
          if ((v[k >> 2] >> (8 * (k & 3))) & 0xFFu) bits |= 1u << k;
        if (n - cl < 16) bits &= (1u << (n - cl)) - 1u;
      }
      if (__builtin_amdgcn_ballot_w64(bits != 0) == 0) continue;   // no kept column here
      const int cnt = __popc(bits);
      int pre = cnt;  // inclusive scan over lanes
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(pre, off);
        if (lane >= off) pre += o;
      }
      const int tot = __shfl(pre, 63);
      if (tot == 0) continue;
      int idx = total + pre - cnt;
      while (bits) {
        const int b = __builtin_ctz(bits);
        bits &= bits - 1;
        const int64_t col = cl + b;
        if (idx < 64) list[w][idx] = (int)col;
        const float z = load1(xr, a.bf16, col) * a.c1;
        if (z > lm) {
          ls = lm == -INFINITY ? 0.f : ls * expf(lm - z);
          lm = z;
        }
        ls += expf(z - lm);
        ++idx;
      }
      total += tot;
    }
  }
  __builtin_amdgcn_wave_barrier();
  float lse = -INFINITY;
  if (total > 0 && total <= 64) {
    const bool live = lane < total;
    const float z = live ? load1(xr, a.bf16, list[w][lane]) * a.c1 : -INFINITY;
    float M;
    const float e = wave_set_sum(z, live, M, pow2_ceil(total));
    lse = M + logf(e);
  } else if (total > 64) {
    float M = lm, S = ls;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float om = __shfl_xor(M, off), os = __shfl_xor(S, off);
      const float N = fmaxf(M, om);
      // Both lanes of a pair form the same two products and add them in lane order.
      const float mine = M == -INFINITY ? 0.f : S * expf(M - N);
      const float other = om == -INFINITY ? 0.f : os * expf(om - N);
      S = (lane & off) ? other + mine : mine + other;
      M = N;
    }
    lse = M + logf(S);
  }
  const int64_t tg = a.targets[row];
  if (tg < 0 || tg >= a.real_vocab) status |= LLP_STATUS_TARGET_OUT_OF_RANGE;
  const int64_t loc = tg - a.offset;
  const bool hit = tg >= 0 && tg < a.real_vocab && loc >= 0 && loc < n && kr[loc] != 0;
  if (lane == 0) {
    const float t = hit ? load1(xr, a.bf16, loc) * a.c1 : 0.f;
    a.out_t[row] = t;
    a.out_f[row] = hit ? 1 : 0;
    a.out_l[row] = lse;
    if (a.out_p) a.out_p[row] = hit ? t - lse : -INFINITY;
    if (status && a.status) atomicOr(a.status, status);
  }
}

hipError_t launch_layout(const LayoutArgs& a, hipStream_t s) {
  const int64_t nb = layout_blocks(a.T);
  if (nb > 1) {
    hipLaunchKernelGGL(k_layout_count, dim3((unsigned)nb), dim3(LAYOUT_THREADS), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_layout, dim3((unsigned)nb), dim3(LAYOUT_THREADS), 0, s, a);
  return hipGetLastError();
}

// The GEMM grids: OVERSUBSCRIBE workgroups per tile, each drawing its tile from the per-XCD
// queues whose counters the layout kernel zeroed.
static inline unsigned workers(int tiles) {
  return (unsigned)(((int64_t)tiles * OVERSUBSCRIBE_NUM + OVERSUBSCRIBE_DEN - 1) / OVERSUBSCRIBE_DEN);
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  if (a.nvt <= 0 || a.ntb <= 0) return hipGetLastError();
  const int64_t ntiles = (int64_t)a.nvt * a.ntb;
  const int n = a.H / KSTEP;
  const dim3 block(64 * FWD_WAVES);
  if (n >= 2 && n % 2 == 0) {
    // One worker per compute unit, at most one per tile, in whole XCD rows.
    int64_t workers = a.workers > 0 && a.workers < ntiles ? a.workers : ntiles;
    workers = (workers + NUM_XCD - 1) / NUM_XCD * NUM_XCD;
    const dim3 grid((unsigned)workers);
    if (a.bias == nullptr) hipLaunchKernelGGL((k_fwd<BIAS_NONE, FWD_WAVES>), grid, block, 0, s, a);
    else if (a.bias_f32) hipLaunchKernelGGL((k_fwd<BIAS_F32, FWD_WAVES>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_fwd<BIAS_BF16, FWD_WAVES>), grid, block, 0, s, a);
  } else {
    const dim3 grid((unsigned)ntiles);
    if (a.bias == nullptr) hipLaunchKernelGGL((k_fwd_tiles<BIAS_NONE, FWD_WAVES>), grid, block, 0, s, a);
    else if (a.bias_f32) hipLaunchKernelGGL((k_fwd_tiles<BIAS_F32, FWD_WAVES>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_fwd_tiles<BIAS_BF16, FWD_WAVES>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int64_t T_cap, hipStream_t s) {
  if (T_cap > 0)
    hipLaunchKernelGGL(k_combine, dim3(ceil_div64(T_cap, COMBINE_ROWS)),
                       dim3(COMBINE_ROWS * COMBINE_CHAINS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  if (a.T > 0) hipLaunchKernelGGL(k_merge, dim3(ceil_div64(a.T, 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topp(const ToppArgs& a, hipStream_t s) {
  if (a.T > 0) hipLaunchKernelGGL(k_topp, dim3(ceil_div64(a.T, 16)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_grad(const GradArgs& a, hipStream_t s) {
  if (a.nvt > 0 && a.ntb > 0)
    hipLaunchKernelGGL(k_grad<GRAD_WAVES>, dim3(workers(a.nvt * a.ntb)),
                       dim3(64 * GRAD_WAVES), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dh(const DhArgs& a, hipStream_t s) {
  const int n = a.ntm * a.ntn * a.nsplit;
  if (n > 0 && a.accumulate) {
    hipLaunchKernelGGL(k_dh_acc<DH_WAVES>, dim3(workers(n)), dim3(64 * DH_WAVES), 0, s, a);
  } else if (n > 0) {
    hipLaunchKernelGGL(k_dh<DH_WAVES>, dim3(workers(n)), dim3(64 * DH_WAVES), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_dh_reduce(const DhReduceArgs& a, hipStream_t s) {
  const int64_t n = a.T * (a.H / 8);
  if (n > 0) hipLaunchKernelGGL(k_dh_reduce, dim3(ceil_div64(n, 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dw(const DwArgs& a, hipStream_t s) {
  const int n = a.ntm * a.ntn;
  if (n > 0) {
    const dim3 grid(workers(n));
    if (a.overwrite) hipLaunchKernelGGL(k_dw<true>, grid, dim3(NTHREADS), 0, s, a);
    else hipLaunchKernelGGL(k_dw<false>, grid, dim3(NTHREADS), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_zero_rows(const ZeroArgs& a, hipStream_t s) {
  const int64_t n = (a.r1 - a.r0) * a.cols;
  if (n > 0) {
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(k_zero_rows, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256),
                       0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_transpose(const TransposeArgs& a, int64_t rows, hipStream_t s) {
  if (rows > 0 && a.cols > 0)
    hipLaunchKernelGGL(k_transpose, dim3((unsigned)(rows / 64), (unsigned)(a.cols / 64)), dim3(256),
                       0, s, a);
  return hipGetLastError();
}

hipError_t launch_dbias(const DbArgs& a, hipStream_t s) {
  if (a.n_real > 0) hipLaunchKernelGGL(k_dbias, dim3(ceil_div64(a.n_real, 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_logits(const LogitsArgs& a, hipStream_t s) {
  if (a.T > 0) hipLaunchKernelGGL(k_logits, dim3((unsigned)a.T), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_keep(const KeepArgs& a, hipStream_t s) {
  if (a.T > 0) hipLaunchKernelGGL(k_keep, dim3((unsigned)((a.T + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// Static scratch for llp_forward_noalloc, the forward for callers that cannot allocate device
// memory. The array is part of the code object, so every device the library is loaded on
// holds its own copy (SCRATCH_BYTES each, until the process ends) at its own address. In host
// code `scratch` names a host-side stand-in, not device memory: the device address is looked
// up once per device with hipGetSymbolAddress (scratch_init, called by llp_open with that
// device current) and only that address is handed to kernels.
// ------------------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];
static void* g_scratch_addr[MAX_DEVICES];

hipError_t scratch_init(int device) {
  if (device < 0 || device >= MAX_DEVICES) return hipErrorInvalidDevice;
  if (g_scratch_addr[device] != nullptr) return hipSuccess;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (p == nullptr) return hipErrorInvalidSymbol;
  g_scratch_addr[device] = p;
  return hipSuccess;
}

void* scratch_address(int device) {
  return device >= 0 && device < MAX_DEVICES ? g_scratch_addr[device] : nullptr;
}

hipError_t probe_kernels() {
  hipFuncAttributes attr;
  return hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(k_fwd<BIAS_NONE, FWD_WAVES>));
}

}  // namespace llp
