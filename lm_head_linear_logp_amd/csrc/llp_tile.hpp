// llp_tile.hpp -- bf16 MFMA tile machinery for gfx950 shared by the fused forward, the
// gradient recompute and the two backward products.
//
// Workgroup tile: BM x BN = 256 x 256 outputs, BK = 64 deep, 256 threads = 4 wave64s in a
// 2 x 2 arrangement, each wave owning a 128 x 128 sub-tile as 4 x 4 blocks of the
// v_mfma_f32_32x32x16_bf16 instruction (256 fp32 accumulators per lane).
//
// Operands are staged through LDS in a K-contiguous layout: a tile row (one M or N index)
// holds BK = 64 bf16 = eight 16-byte chunks; chunk c of row r sits at chunk slot
// c ^ swz(r), which spreads both the 16-byte writes and the MFMA operand reads over all LDS
// banks. Two LDS stages (2 x 64 KiB) double-buffer the K loop: global loads for step s+1 are
// in flight while the MFMAs of step s run, then written to the other stage; one barrier per
// step.
//
// Two global loaders fill a stage:
//   LdK  -- rows along M (or N), K contiguous in memory: 16-byte chunk loads.
//   LdMN -- rows along K, M (or N) contiguous in memory: each thread loads an 8 x 8 bf16
//           block (8 K-rows x 16 bytes) and transposes it in registers, so the LDS tile is
//           K-contiguous either way and the MFMA loop is shared.
//
// MFMA 32x32x16 bf16 lane layout (per the CDNA4 ISA): lane l supplies A[i][k] and B[k][j]
// for i, j = l % 32 and k = 8 * (l / 32) + 0..7; accumulator register r of lane l holds
// D[i][j] with j = l % 32 and i = 8 * (r / 4) + 4 * (l / 32) + r % 4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int NTHREADS = 256;
constexpr int STAGE_ELEMS = BM * BK;              // bf16 elements per operand stage
constexpr int MAIN_LDS_BYTES = 4 * STAGE_ELEMS * 2;  // A0 B0 A1 B1 = 128 KiB
constexpr int NUM_XCD = 8;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// Accumulator register r of lane `lane` in the 32x32 block holds this row (0..31).
__device__ __forceinline__ int mfma_row(int r, int lane) {
  return ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3);
}

// Hardware dispatch places workgroup b on XCD b % 8. Remap so that each XCD runs a
// contiguous range of logical tiles (bijective for any n).
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int full = n / NUM_XCD, rem = n % NUM_XCD;
  const int x = b % NUM_XCD, i = b / NUM_XCD;
  return x * full + (x < rem ? x : rem) + i;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// K-contiguous loader: thread t owns chunk (t & 7) of rows (t >> 3) + 32 * i, i = 0..7.
struct LdK {
  const uint16_t* p[8];  // row pointers, already offset by the thread's chunk
  u32x4 v[8];

  __device__ __forceinline__ void load(int kstep) {
    const int k0 = kstep * BK;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const u32x4*>(p[i] + k0);
  }
  __device__ __forceinline__ void store(uint16_t* s) const {
    const int t = threadIdx.x, c = t & 7, r0 = t >> 3;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = r0 + 32 * i;
      *reinterpret_cast<u32x4*>(s + r * BK + ((c ^ swz(r)) << 3)) = v[i];
    }
  }
};

// M/N-contiguous loader with in-register 8x8 transpose. Thread t owns the block of K-rows
// 8 * (t >> 5) + 0..7 and M/N columns 8 * (t & 31) + 0..7 of the stage. `RowPtr` maps a
// K index to the address of that row's 8 columns, or nullptr for a zero row.
template <class RowPtr>
struct LdMN {
  RowPtr rp;
  u32x4 v[8];

  __device__ __forceinline__ void load(int kstep) {
    const int kb = threadIdx.x >> 5;
    const int k0 = kstep * BK + kb * 8;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint16_t* q = rp(k0 + u);
      v[u] = q ? *reinterpret_cast<const u32x4*>(q) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(uint16_t* s) const {
    const int kb = threadIdx.x >> 5, mb = threadIdx.x & 31;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // Column i of the 8x8 block: K-rows 0..7 packed two per dword.
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t lo = v[2 * d][i >> 1], hi = v[2 * d + 1][i >> 1];
        o[d] = (i & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
      }
      const int r = mb * 8 + i;
      *reinterpret_cast<u32x4*>(s + r * BK + ((kb ^ swz(r)) << 3)) = o;
    }
  }
};

// Per-lane LDS read offsets of the wave's 4 A rows and 4 B rows.
struct Frag {
  int aoff[4], at[4], boff[4], bt[4];
  __device__ __forceinline__ void init(int wm, int wn, int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = wm * 128 + i * 32 + (lane & 31);
      const int rb = wn * 128 + i * 32 + (lane & 31);
      aoff[i] = ra * BK;
      at[i] = (lane >> 5) ^ swz(ra);
      boff[i] = rb * BK;
      bt[i] = (lane >> 5) ^ swz(rb);
    }
  }
};

__device__ __forceinline__ void mma_stage(const uint16_t* As, const uint16_t* Bs,
                                          const Frag& f, f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = *reinterpret_cast<const bf16x8*>(As + f.aoff[i] + (((2 * kk) ^ f.at[i]) << 3));
      b[i] = *reinterpret_cast<const bf16x8*>(Bs + f.boff[i] + (((2 * kk) ^ f.bt[i]) << 3));
    }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
  }
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
}

// acc += A[M-tile, K-steps ks0..ks1) . B[N-tile, same]^T, K steps in ascending order.
// Branch-free body (stage chosen by address arithmetic, last step peeled) so that the
// accumulators stay in place across iterations.
template <class LA, class LB>
__device__ __forceinline__ void mainloop(LA& la, LB& lb, int ks0, int ks1, uint16_t* smem,
                                         f32x16 (&acc)[4][4]) {
  const int n = ks1 - ks0;
  if (n <= 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  Frag f;
  f.init(wave & 1, wave >> 1, lane);
  // Stage s: A at smem + (s & 1) * 2 * STAGE_ELEMS, B right after it.
  la.load(ks0);
  lb.load(ks0);
  la.store(smem);
  lb.store(smem + STAGE_ELEMS);
  __syncthreads();
  for (int s = 0; s < n - 1; ++s) {
    la.load(ks0 + s + 1);
    lb.load(ks0 + s + 1);
    const uint16_t* cur = smem + (s & 1) * (2 * STAGE_ELEMS);
    uint16_t* nxt = smem + ((s + 1) & 1) * (2 * STAGE_ELEMS);
    mma_stage(cur, cur + STAGE_ELEMS, f, acc);
    la.store(nxt);
    lb.store(nxt + STAGE_ELEMS);
    __syncthreads();
  }
  const uint16_t* last = smem + ((n - 1) & 1) * (2 * STAGE_ELEMS);
  mma_stage(last, last + STAGE_ELEMS, f, acc);
  __syncthreads();
}

}  // namespace llp
