// llp_tile.hpp -- the bf16 MFMA GEMM tile for gfx950 shared by the fused forward, the
// gradient recompute and the two backward products.
//
// Workgroup tile: BM x BN = 256 x 256 outputs. With 4 wave64s (2 x 2, one per SIMD) each wave
// owns a 128 x 128 sub-tile as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators
// per lane, held in AGPRs); with 8 wave64s (2 x 4, two per SIMD, the forward) each owns
// 128 x 64 as 4 x 2 blocks (128 accumulators), NFB = 2 fragments of B. The stages, the DMA
// pattern and every output's MFMA chain are the same either way. Operands are read either
// K-contiguous ([rows][K], K innermost) or K-major, through direct global->LDS loads (dma::
// below).
//
// MFMA 32x32x16 bf16 lane layout (CDNA4 ISA): lane l supplies A[i][k] and B[k][j] for
// i, j = l % 32 and k = 8 * (l / 32) + 0..7; accumulator register r of lane l holds D[i][j]
// with j = l % 32 and i = 8 * (r / 4) + 4 * (l / 32) + r % 4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int NTHREADS = 256;
constexpr int NUM_XCD = 8;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

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

// Work distribution over the XCDs for the backward GEMM kernels. The XCDs of one chip run at
// different clocks under load (measured 1.60-1.80 GHz within one launch), so equal shares of
// tiles per XCD leave the fast ones idle while the slowest finishes. Hardware dispatch puts
// workgroup b on XCD b % 8 and each XCD starts its share of the grid in order (b / 8) as its
// CUs free up. XCD x owns the contiguous range of logical tiles xcd_remap gives it (its
// queue), so the CUs of an XCD run consecutive tiles that share operand slices in its L2. The
// first 3/4 of a queue go to the XCD's workgroups by position, with no synchronisation; the
// last quarter is handed out in order through a counter, to the XCD's later workgroups and,
// once it runs dry, to other XCDs' workgroups that have emptied their own. The grid holds
// OVERSUBSCRIBE workgroups per tile, so a faster XCD runs more workgroups and so more tiles; a
// workgroup that finds every queue empty exits. Which workgroup runs a tile changes nothing in
// that tile's arithmetic: results are bitwise those of any other assignment. (The forward
// runs persistent workers over the same static order instead: there the dynamic tail
// measured ~5% slower, the backward kernels ~2% faster.)
constexpr int OVERSUBSCRIBE_NUM = 5, OVERSUBSCRIBE_DEN = 4;   // workgroups per tile: 1.25
// A launch's counters (QCTR_INTS of them, llp_internal.h): [0, 8) the queues' dynamic parts,
// [8] set once every queue is empty.

__device__ __forceinline__ int queue_first(int n, int x) {
  const int full = n / NUM_XCD, rem = n % NUM_XCD;
  return x * full + (x < rem ? x : rem);
}
__device__ __forceinline__ int queue_size(int n, int x) {
  return n / NUM_XCD + (x < n % NUM_XCD ? 1 : 0);
}
__device__ __forceinline__ int queue_static(int size) { return size - (size + 3) / 4; }

// One dynamic tile of n for a workgroup on XCD x, or -1 when every queue's dynamic part is
// empty: global atomic operations (vector memory) on ctr[0..8] (zero at the launch), own XCD's
// queue first. Called by one thread.
__device__ __forceinline__ int claim_dynamic(int* ctr, int n, int x) {
  int t = -1;
  int k = atomicAdd(ctr + x, 1);
  if (k < queue_size(n, x) - queue_static(queue_size(n, x))) {
    t = queue_first(n, x) + queue_static(queue_size(n, x)) + k;
  } else if (atomicOr(ctr + NUM_XCD, 0) == 0) {
    for (int d = 1; d < NUM_XCD && t < 0; ++d) {
      const int y = (x + d) % NUM_XCD;
      const int sy = queue_static(queue_size(n, y));
      k = atomicAdd(ctr + y, 1);
      if (k < queue_size(n, y) - sy) t = queue_first(n, y) + sy + k;
    }
    if (t < 0) atomicOr(ctr + NUM_XCD, 1);
  }
  return t;
}

// The workgroup's logical tile of n, or -1 when every queue is empty. Called by every thread
// (the static branch is uniform). A dynamic tile is claimed by thread 0 and reaches the other
// threads through `slot`, a word of the pipeline's LDS (a separate __shared__ word would be a
// second LDS object, and with two the compiler no longer tells the stages' DMA writes from
// the fragment reads: it waits for every DMA load before each read, measured 62% slower).
__device__ __forceinline__ int take_tile(int* ctr, int n, int* slot) {
  const int x = blockIdx.x % NUM_XCD, i = blockIdx.x / NUM_XCD;
  const int s0 = queue_static(queue_size(n, x));
  if (i < s0) return queue_first(n, x) + i;
  if (threadIdx.x == 0) *slot = claim_dynamic(ctr, n, x);
  __syncthreads();
  const int t = *slot;
  __syncthreads();   // the slot sits in the pipeline's LDS, which the first DMA overwrites
  return t;
}

// Logical tile -> (vocabulary tile, token block) for the vocabulary x token grids. Tiles
// run in groups of VG vocabulary tiles x all token blocks, token block slowest within a group:
// with VG = 8 the 32 workgroups an XCD runs at once cover 8 vocabulary tiles x 4 token blocks,
// whose operands (8 weight + 4 hidden tiles, 24 MiB) are each fetched once into that XCD's L2
// per round. Bijective for any grid. VG is per kernel: 8 for the forward, the gradient tile
// and dhidden; 4 for dweight (4 vocabulary x 8 hidden tiles per round measured ~1.7% faster
// there and 2% slower for the forward). The order changes no tile's arithmetic.
constexpr int VOCAB_GROUP = 8;
template <int VG = VOCAB_GROUP>
__device__ __forceinline__ void vocab_token_tile(int tile, int nvt, int ntb, int& vt, int& tb) {
  const int grp = tile / (VG * ntb), gi = tile % (VG * ntb);
  const int rest = nvt - grp * VG;
  const int gsz = rest < VG ? rest : VG;
  vt = grp * VG + gi % gsz;
  tb = gi / gsz;
}

// Two floats to packed bf16 (first in the low half), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Read one accumulator into a VGPR at the point of use. Pinning the operand to an AGPR
// keeps the register allocator from moving accumulators into VGPRs for the whole K loop
// (which spills) when an epilogue feeds them to vector ALU instructions.
__device__ __forceinline__ float acc_read(float x) {
  float r;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(x));
  return r;
}

template <int NFB>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][NFB]) {
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < NFB; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
}

// ------------------------------------------------------------------------------------
// DMA pipeline for operands that are K-contiguous in memory. K step BKD = 64 (128 bytes per
// row: one whole L2 line, so a load instruction's requests are full lines; with 64-byte row
// pieces the L1's request rate, not bandwidth, caps the stream below what the MFMAs need).
// NST = 2 LDS stages of 2 x 32 KiB. One instruction moves 64 lanes x 16 bytes into a
// contiguous 1 KiB LDS window in lane order: 8 rows of 8 chunks. With NW waves, wave w fills
// rows R w .. R w + R - 1 (R = 256 / NW) of each operand with R / 8 instructions; lane i of
// instruction u lands in row R w + 8u + i/8 at slot i%8 and so fetches that row's logical
// chunk (i%8) ^ swz8(row).
// swz8 puts 8 (and 16) consecutive rows reading one logical chunk on distinct banks.
// ------------------------------------------------------------------------------------
namespace dma {

constexpr int BKD = 64;
constexpr int NST = 2;
constexpr int NI = 8;            // load instructions per wave per operand per step, 4 waves
constexpr int STAGE = BM * BKD;  // bf16 elements per operand per stage
constexpr int LDS_BYTES = NST * 2 * STAGE * 2;

__device__ __forceinline__ int swz8(int row) { return (row ^ (row >> 3)) & 7; }

// One operand's loads: a buffer resource whose base is the operand's first row in the tile, and
// per load instruction this lane's 32-bit byte offset at K step 0; the K step's offset goes in
// the instruction's scalar offset. Offsets are exact (rows clamped by the caller), so every
// access lies inside [base, base + bytes), the range given to the resource. With NW waves a
// wave fills 256 / NW rows of each operand with NIW = 32 / NW instructions.
// The buffer resource and the DMA instruction, outside the loader template (non-template
// functions, like the rest of the device code, are parsed once; the host pass rejects these
// builtins inside a class template's instantiation).
struct BufRsrc {
  __amdgpu_buffer_rsrc_t rsrc;
  // Raw buffer (stride 0) over `bytes` bytes from `base` (gfx9 resource word 3: 32-bit data).
  __device__ __forceinline__ void init(const uint16_t* base, uint64_t bytes) {
    rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0,
                                             (int)(uint32_t)(bytes < 0xFFFFFFFFull ? bytes : 0xFFFFFFFFull),
                                             0x00020000);
  }
  // 16 bytes per lane from byte offset voff + soff into the LDS window at `lds` (lane order).
  __device__ __forceinline__ void load_lds(uint16_t* lds, uint32_t voff, int soff) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16,
                                             voff, soff, 0, 0);
  }
};

template <int NW>
struct LoaderT : BufRsrc {
  static constexpr bool KMAJOR = false;
  static constexpr int NIW = 32 / NW;
  static constexpr int RPW = BM / NW;  // rows per wave
  uint32_t voff[NIW];

  __device__ __forceinline__ static int row_of(int u) {
    return RPW * (threadIdx.x >> 6) + 8 * u + ((threadIdx.x & 63) >> 3);
  }
  __device__ __forceinline__ static int chunk_of(int u) {
    return (threadIdx.x & 7) ^ swz8(row_of(u));
  }
  // Instruction u reads row `row` (relative to the base, row stride `ld` elements) for this lane.
  __device__ __forceinline__ void set(int u, int64_t row, int64_t ld) {
    voff[u] = (uint32_t)((row * ld + chunk_of(u) * 8) * 2);
  }
  // One DMA instruction (u = 0..NIW-1) of this wave for K step `kstep` into `stage`.
  __device__ __forceinline__ void issue1(uint16_t* stage, int kstep, int u) const {
    // The wave index is uniform: keep the LDS destination (M0) in scalar registers.
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    load_lds(stage + (RPW * w + 8 * u) * BKD, voff[u], kstep * (BKD * 2));
  }
};
using Loader = LoaderT<4>;

// A K-major operand ([K][cols] in memory, the tile's columns contiguous): a stage holds the K
// step's 64 rows x 256 columns, 512 bytes per K-row, and 16-byte chunk c of K-row r sits at
// chunk c ^ fk(r). One instruction fills two K-rows; wave w fills K-rows 16w .. 16w+15 with 8
// instructions, lane i of instruction u landing in K-row 16w + 2u + i/32 at chunk i%32.
// The resource is rebased at every K step (its base is that step's first row), so offsets stay
// small for any number of rows; rows past `maxrow` (the last readable one) are read as maxrow
// and columns past the valid ones as column 0 (callers never use those values).
// The swizzle spreads one transposing fragment read (FragOp<true>) over every LDS bank: its 64
// lanes read 8 bytes each from K-rows 8(g/2) + j (g = lane/16, j = lane/4 % 4) at chunks
// C + 2(g%2) + (lane/2 % 2), so XOR-ing the chunk with 4j + 16(g/2) gives the 64 lanes 64
// distinct 8-byte slots of a 512-byte window: each of the 64 four-byte banks is read twice,
// the minimum for 512 bytes. (XOR-ing with 2j alone left pairs of lanes on one bank in every
// half-wave.)
__device__ __forceinline__ int fk(int r) { return 4 * (r & 3) + 16 * ((r >> 3) & 1); }

// One K-major DMA instruction (non-template, like BufRsrc): the resource is based at K step
// `kstep`'s first row, 16 bytes per lane from byte offset voff into the LDS window at `lds`.
__device__ __forceinline__ void loadk_issue(const uint16_t* base, int64_t ld, int kstep,
                                            uint16_t* lds, uint32_t voff) {
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(base + (int64_t)kstep * BKD * ld), (short)0, (int)(BKD * ld * 2), 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, 0, 0, 0);
}

// With NW waves, wave w fills K-rows KR w .. KR w + KR - 1 (KR = 64 / NW) of a stage with KR / 2
// instructions, two K-rows each.
template <int NW>
struct LoaderKT {
  static constexpr bool KMAJOR = true;
  static constexpr int KR = BKD / NW;  // K-rows per wave
  static constexpr int NIW = KR / 2;
  const uint16_t* base;  // row 0, first column of the tile
  int64_t ld;            // row stride (elements)
  int maxrow;            // last readable row
  int r0;                // this lane's K-row for u = 0 within a step: KR w + lane/32
  int cb[NIW];           // byte offset of this lane's source chunk for instruction u

  __device__ __forceinline__ void init(const uint16_t* b, int64_t ld_, int maxrow_, int ncols) {
    base = b;
    ld = ld_;
    maxrow = maxrow_;
    const int lane = threadIdx.x & 63;
    r0 = KR * (threadIdx.x >> 6) + (lane >> 5);
#pragma unroll
    for (int u = 0; u < NIW; ++u) {
      // Position lane % 32 of the stage's K-row r0 + 2u holds chunk (lane % 32) ^ fk(r0 + 2u).
      int c = (lane & 31) ^ fk(r0 + 2 * u);
      if (8 * c >= ncols) c = 0;
      cb[u] = 16 * c;
    }
  }
  __device__ __forceinline__ void issue1(uint16_t* stage, int kstep, int u) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rlim = maxrow - kstep * BKD;
    const int r = r0 + 2 * u < rlim ? r0 + 2 * u : rlim;
    loadk_issue(base, ld, kstep, stage + (KR * w + 2 * u) * BM, (uint32_t)(r * (int)ld * 2 + cb[u]));
  }
};
using LoaderK = LoaderKT<4>;

// Fragment addressing of one operand in a stage. Row-major (K-contiguous) operands read one
// 16-byte chunk per fragment; K-major operands build it from two ds_read_b64_tr_b16, which
// transpose within each 16-lane group: source lane 4j + t reads 4 columns (quad t) of K-row j,
// and output lane i receives those 4 K-rows of column i (element i % 4 of source lanes i/4,
// 4 + i/4, 8 + i/4, 12 + i/4). MFMA lane l needs column l % 32 and K = 8(l/32) + 0..7, so
// group g = l/16 covers columns 16(g%2) .. +15 and K-rows 8(g/2) .. +7 in two reads.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

template <bool KMAJ, int NF = 4>
struct FragOp;

// NF fragments of 32 rows from row r0 of the stage.
template <int NF>
struct FragOp<false, NF> {
  int off[NF], t[NF];
  __device__ __forceinline__ void init_rows(int r0, int lane) {
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int r = r0 + i * 32 + (lane & 31);
      off[i] = r * BKD;
      t[i] = (lane >> 5) ^ swz8(r);
    }
  }
  __device__ __forceinline__ void init(int wx, int lane) { init_rows(wx * 32 * NF, lane); }
  // The whole fragment (h must be 0).
  __device__ __forceinline__ bf16x8 read(const uint16_t* st, int kk, int i) const {
    return *reinterpret_cast<const bf16x8*>(st + off[i] + (((2 * kk) ^ t[i]) << 3));
  }
};

// NF fragments of 32 columns from column 32 NF wx of the stage.
template <int NF>
struct FragOp<true, NF> {
  int off[NF];  // bytes
  __device__ __forceinline__ void init(int wx, int lane) {
    const int g = lane >> 4, j = (lane >> 2) & 3, t = lane & 3;
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int chunk = wx * 4 * NF + 4 * i + 2 * (g & 1) + (t >> 1);
      const int row = 8 * (g >> 1) + j;   // fk of every K-row this lane reads is fk(row)
      off[i] = row * (BM * 2) + 16 * (chunk ^ fk(row)) + 8 * (t & 1);
    }
  }
  // K-rows 16kk + 8(g/2) + 4h .. +3 of this lane's column.
  __device__ __forceinline__ v4i16 read_half(const uint16_t* st, int kk, int i, int h) const {
    return tr_read(reinterpret_cast<const unsigned char*>(st) + off[i] + (16 * kk + 4 * h) * (BM * 2));
  }
  // A restrict-qualified pointer gives the read an alias scope, so the compiler need not make
  // it wait for DMA into the other stage.
  static __device__ __forceinline__ v4i16 tr_read(const unsigned char* __restrict__ p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
  }
  __device__ __forceinline__ bf16x8 read(const uint16_t* st, int kk, int i) const {
    const v4i16 lo = read_half(st, kk, i, 0), hi = read_half(st, kk, i, 1);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

// A wave's sub-tile: 4 fragments (128 rows) of A at wm * 128, NFB fragments of B at
// wn * 32 * NFB.
template <bool AK, bool BK, int NFB = 4>
struct Frag {
  FragOp<AK> a;
  FragOp<BK, NFB> b;
  __device__ __forceinline__ void init(int wm, int wn, int lane) {
    a.init(wm, lane);
    b.init(wn, lane);
  }
};

// Fragments of 16-deep substep kk (0..3): lane l holds k = 16kk + 8(l/32) + 0..7.
template <bool AK, bool BK, int NFB>
__device__ __forceinline__ void load_frag(const uint16_t* As, const uint16_t* Bs,
                                          const Frag<AK, BK, NFB>& f, int kk, bf16x8 (&a)[4],
                                          bf16x8 (&b)[NFB]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = f.a.read(As, kk, i);
    if (i < NFB) b[i] = f.b.read(Bs, kk, i);
  }
}

// MFMAs number lo..hi-1 of one 16-deep substep, in (mi, ni) row-major order.
template <int LO, int HI, int NFB>
__device__ __forceinline__ void mfmas(const bf16x8 (&a)[4], const bf16x8 (&b)[NFB],
                                      f32x16 (&acc)[4][NFB]) {
#pragma unroll
  for (int k = LO; k < HI; ++k)
    acc[k / NFB][k % NFB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k / NFB], b[k % NFB],
                                                                   acc[k / NFB][k % NFB], 0, 0, 0);
}

// Wait until at most n of this wave's vector-memory instructions are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt at maxima).
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier that orders LDS only: this wave's LDS reads have returned (lgkmcnt 0)
// before any wave passes. __syncthreads() would also drain every vector-memory load,
// including the DMA loads still in flight for later steps. The memory clobber keeps the
// compiler from moving memory accesses across it; DMA completion is waited for explicitly.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// sched_group_barrier masks (LLVM AMDGPU): MFMA, VMEM read, DS read.
constexpr int SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100;

// Issue DMA instructions LO..HI-1 of one K step (instruction i: operand i&1, slot i>>1).
template <int LO, int HI, class LA, class LB>
__device__ __forceinline__ void issue_range(const LA& la, const LB& lb, uint16_t* stage, int kstep) {
#pragma unroll
  for (int i = LO; i < HI; ++i) {
    if (i & 1) lb.issue1(stage + STAGE, kstep, i >> 1);
    else la.issue1(stage, kstep, i >> 1);
  }
}

// Schedule of one region: 16 MFMAs, NR fragment reads one per MFMA from the first, and D DMA
// instructions spread evenly over the 16 MFMAs.
template <int D, int NR, int I, int NM>
__device__ __forceinline__ void region_slot() {
  __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
  if constexpr (I < NR) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
  constexpr int nv = ((I + 1) * D) / NM - (I * D) / NM;
  if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, nv, 0);
  if constexpr (I + 1 < NM) region_slot<D, NR, I + 1, NM>();
}

// Memory instructions of one region in slot order (the compiler keeps LDS reads and DMA
// writes in program order, so the source order is the issue order). Reads go fragment by
// fragment, A then B, one or two reads each (row-major or K-major); DMA instructions
// QB + (I*D)/16 .. of step `kstep` into `dst` follow in their slots.
template <bool AK, bool BK, int NFB>
struct ReadPlan {
  static constexpr int RA = AK ? 2 : 1, RB = BK ? 2 : 1;
  static constexpr int NR = 4 * RA + NFB * RB;
  static constexpr int NM = 4 * NFB;  // MFMAs per region
  // Reads of fragment i (A, then B while i < NFB), and the first read slot of fragment i.
  static constexpr int per(int i) { return RA + (i < NFB ? RB : 0); }
  static constexpr int start(int i) { return i == 0 ? 0 : start(i - 1) + per(i - 1); }
  static constexpr int frag(int I, int i = 0) { return I < start(i + 1) ? i : frag(I, i + 1); }
};

template <int D, int QB, int I, bool AK, bool BK, int NFB, class LA, class LB>
__device__ __forceinline__ void region_mem(const LA& la, const LB& lb, const uint16_t* st,
                                           const Frag<AK, BK, NFB>& f, int kk, bf16x8 (&na)[4],
                                           bf16x8 (&nb)[NFB], v4i16 (&tmp)[4], uint16_t* dst,
                                           int kstep) {
  using P = ReadPlan<AK, BK, NFB>;
  if constexpr (I < P::NR) {
    constexpr int i = P::frag(I), r = I - P::start(i);
    if constexpr (r < P::RA) {
      if constexpr (!AK) {
        na[i] = f.a.read(st, kk, i);
      } else if constexpr (r == 0) {
        tmp[i] = f.a.read_half(st, kk, i, 0);
      } else {
        const v4i16 hi = f.a.read_half(st, kk, i, 1);
        na[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(tmp[i], hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    } else {
      constexpr int rb = r - P::RA;
      if constexpr (!BK) {
        nb[i] = f.b.read(st + STAGE, kk, i);
      } else if constexpr (rb == 0) {
        tmp[i] = f.b.read_half(st + STAGE, kk, i, 0);
      } else {
        const v4i16 hi = f.b.read_half(st + STAGE, kk, i, 1);
        nb[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(tmp[i], hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  }
  issue_range<QB + (I * D) / P::NM, QB + ((I + 1) * D) / P::NM>(la, lb, dst, kstep);
  if constexpr (I + 1 < P::NM)
    region_mem<D, QB, I + 1, AK, BK, NFB>(la, lb, st, f, kk, na, nb, tmp, dst, kstep);
}

// One region: 4 x NFB MFMAs on (a, b); fragment reads of substep kk from stage `st` into
// (na, nb); DMA instructions QB .. QB+D-1 of step `kstep` into stage `dst`.
template <int D, int QB, bool AK, bool BK, int NFB, class LA, class LB>
__device__ __forceinline__ void region(const LA& la, const LB& lb, const bf16x8 (&a)[4],
                                       const bf16x8 (&b)[NFB], const uint16_t* st,
                                       const Frag<AK, BK, NFB>& f, int kk, bf16x8 (&na)[4],
                                       bf16x8 (&nb)[NFB], uint16_t* dst, int kstep,
                                       f32x16 (&acc)[4][NFB]) {
  using P = ReadPlan<AK, BK, NFB>;
  v4i16 tmp[4];
  mfmas<0, P::NM, NFB>(a, b, acc);
  region_mem<D, QB, 0, AK, BK, NFB>(la, lb, st, f, kk, na, nb, tmp, dst, kstep);
  region_slot<D, P::NR, 0, P::NM>();
  __builtin_amdgcn_sched_barrier(0);
}

// acc += A[M-tile, K-steps ks0..ks1) . B[N-tile, same]^T in ascending K order. LA/LB are Loader
// (row-major, K-contiguous) or LoaderK (K-major); the fragment layout follows.
// Step s (stage s%2) runs four 16-deep substeps in four branch-free regions; fragments
// alternate between two register sets and each region reads the next substep's:
//   R1:     MFMAs of kk0, reads of kk1, DMA of step s+1 (its last NIW loads)
//   R2, R3: MFMAs of kk1, kk2, reads of kk2, kk3
//   -- wait for step s+1's DMA, barrier (every wave is done reading stage s%2) --
//   R4:     MFMAs of kk3, reads of kk0 of step s+1, DMA of step s+2 (its first NIW loads)
// A region holds 4 x NFB MFMAs. A wave's 2 NIW loads of a step (16 with 4 waves, 8 with 8)
// are split over two regions, one per two MFMAs: issued in one burst they
// back up the address unit, and the in-order issue stalls the MFMAs queued behind them. DMA
// steps past the end are clamped to the last step (an in-bounds reload into a stage that is
// never read again), which keeps every iteration the same shape. All DMA is drained before
// returning.
template <class LA, class LB, int NFB = 4>
__device__ __forceinline__ void mainloop(const LA& la, const LB& lb, int ks0, int ks1,
                                         uint16_t* smem, f32x16 (&acc)[4][NFB]) {
  constexpr bool AK = LA::KMAJOR, BK = LB::KMAJOR;
  static_assert(LA::NIW == LB::NIW, "both operands take the same loads per wave");
  constexpr int NIW = LA::NIW;
  constexpr int NQ = 2 * NIW, Q4 = NIW, Q1 = NIW;  // loads per step: NIW in R4, NIW in R1
  const int n = ks1 - ks0;
  if (n <= 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  Frag<AK, BK, NFB> f;
  f.init(wave & 1, wave >> 1, lane);
  const int k1 = ks0 + (1 < n ? 1 : 0);
  issue_range<0, NQ>(la, lb, smem, ks0);
  issue_range<0, Q4>(la, lb, smem + 2 * STAGE, k1);
  wait_vmem_le<Q4>();
  lds_barrier();
  bf16x8 a0[4], b0[NFB], a1[4], b1[NFB];
  load_frag(smem, smem + STAGE, f, 0, a0, b0);
  for (int s = 0; s < n; ++s) {
    uint16_t* cur = smem + (s & 1) * 2 * STAGE;
    uint16_t* nx = smem + ((s + 1) & 1) * 2 * STAGE;
    const int kn = ks0 + (s + 1 < n ? s + 1 : n - 1);
    const int kd = ks0 + (s + 2 < n ? s + 2 : n - 1);
    region<Q1, Q4>(la, lb, a0, b0, cur, f, 1, a1, b1, nx, kn, acc);
    region<NQ - Q4 - Q1, Q4 + Q1>(la, lb, a1, b1, cur, f, 2, a0, b0, nx, kn, acc);
    region<0, 0>(la, lb, a0, b0, cur, f, 3, a1, b1, nx, kn, acc);
    wait_vmem_le<0>();
    lds_barrier();
    region<Q4, 0>(la, lb, a1, b1, nx, f, 0, a0, b0, cur, kd, acc);
  }
  wait_vmem_le<0>();
  __syncthreads();
}

// One K step of mainloop with its loaders made explicit: the DMA slots for step s+1 (regions
// 1-3) take (ln, lbn) at K step kn, those for step s+2 (region 4) take (ld, lbd) at kd.
template <class LA, class LB, int NFB, bool AK, bool BK>
__device__ __forceinline__ void chain_step(const LA& ln, const LB& lbn, int kn, const LA& ld,
                                           const LB& lbd, int kd, uint16_t* cur, uint16_t* nx,
                                           const Frag<AK, BK, NFB>& f, bf16x8 (&a0)[4],
                                           bf16x8 (&b0)[NFB], bf16x8 (&a1)[4], bf16x8 (&b1)[NFB],
                                           f32x16 (&acc)[4][NFB]) {
  constexpr int NIW = LA::NIW;
  constexpr int NQ = 2 * NIW, Q4 = NIW, Q1 = NIW;
  region<Q1, Q4>(ln, lbn, a0, b0, cur, f, 1, a1, b1, nx, kn, acc);
  region<NQ - Q4 - Q1, Q4 + Q1>(ln, lbn, a1, b1, cur, f, 2, a0, b0, nx, kn, acc);
  region<0, 0>(ln, lbn, a0, b0, cur, f, 3, a1, b1, nx, kn, acc);
  wait_vmem_le<0>();
  lds_barrier();
  region<Q4, 0>(ld, lbd, a1, b1, nx, f, 0, a0, b0, cur, kd, acc);
}

// mainloop over K steps 0..n-1 of one tile of a persistent worker (n even, n >= 2): the same
// steps, schedule and arithmetic, with two differences at the tile's edges.
//  - `primed`: the tile's step 0 and the first half of its step 1 are already in flight
//    (issued by the previous tile's call), so the call starts by waiting for them.
//  - The DMA slots past the tile's last step take the next tile's steps 0 and 1 through
//    (la2, lb2). The call then returns with them in flight, and they land while this tile's
//    epilogue runs. With no next tile, the caller passes this tile's loaders as (la2, lb2) and
//    `more` false: the slots reload the last step (as in mainloop) and all DMA is drained
//    before returning.
// The epilogue must not use the two stages (the next tile's loads land there).
template <class LA, class LB, int NFB>
__device__ __forceinline__ void mainloop_chain(const LA& la, const LB& lb, const LA& la2,
                                               const LB& lb2, bool primed, bool more, int n,
                                               uint16_t* smem, f32x16 (&acc)[4][NFB]) {
  constexpr bool AK = LA::KMAJOR, BK = LB::KMAJOR;
  static_assert(LA::NIW == LB::NIW, "both operands take the same loads per wave");
  constexpr int NQ = 2 * LA::NIW, Q4 = LA::NIW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  Frag<AK, BK, NFB> f;
  f.init(wave & 1, wave >> 1, lane);
  if (!primed) {
    issue_range<0, NQ>(la, lb, smem, 0);
    issue_range<0, Q4>(la, lb, smem + 2 * STAGE, 1);
    wait_vmem_le<Q4>();
  } else {
    // The previous epilogue's stores and this tile's setup loads are counted too.
    wait_vmem_le<0>();
  }
  lds_barrier();
  bf16x8 a0[4], b0[NFB], a1[4], b1[NFB];
  load_frag(smem, smem + STAGE, f, 0, a0, b0);
  uint16_t* const s0 = smem;
  uint16_t* const s1 = smem + 2 * STAGE;
  for (int s = 0; s < n - 2; s += 2) {
    chain_step(la, lb, s + 1, la, lb, s + 2, s0, s1, f, a0, b0, a1, b1, acc);
    chain_step(la, lb, s + 2, la, lb, s + 3, s1, s0, f, a0, b0, a1, b1, acc);
  }
  // Steps n-2 (stage 0) and n-1 (stage 1), straight-line (a branch here costs the compiler
  // its in-place accumulators).
  const int k0 = more ? 0 : n - 1, k1 = more ? 1 : n - 1;
  chain_step(la, lb, n - 1, la2, lb2, k0, s0, s1, f, a0, b0, a1, b1, acc);
  chain_step(la2, lb2, k0, la2, lb2, k1, s1, s0, f, a0, b0, a1, b1, acc);
  if (!more) {
    wait_vmem_le<0>();
    __syncthreads();
  }
}

}  // namespace dma

}  // namespace llp
