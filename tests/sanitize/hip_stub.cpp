// hip_stub.cpp -- a host-only stand-in for the HIP runtime and the kernel launchers, so that the
// C-ABI host code (request validation, workspace layout, launch sequences) can be built with the
// host compiler's address and undefined-behaviour sanitizers and run without a GPU.
//
// The stand-in device is one gfx950 GPU with 256 CUs. Each launcher, instead of launching a
// kernel, touches the first and the last element of every array the kernel would address,
// given the launch's arguments (the extent each kernel's indexing reaches). The test driver
// hands the library exactly sized host allocations, so an extent that overruns its buffer (a
// workspace region laid out too small, an output indexed past T) is an out-of-bounds access that
// the address sanitizer reports.
#include <hip/hip_runtime_api.h>
#include <string.h>

#include <vector>

#include "llp_internal.h"

extern "C" {
hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
hipError_t hipGetDeviceCount(int* n) { *n = 1; return hipSuccess; }
hipError_t hipSetDevice(int d) { return d == 0 ? hipSuccess : hipErrorInvalidDevice; }
const char* hipGetErrorString(hipError_t) { return "stub"; }
}
#if HIP_VERSION_MAJOR >= 6
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_t* p, int d) {
#else
hipError_t hipGetDeviceProperties(hipDeviceProp_t* p, int d) {
#endif
  if (d != 0) return hipErrorInvalidDevice;
  memset(p, 0, sizeof(*p));
  strcpy(p->gcnArchName, "gfx950:sramecc+:xnack-");
  p->multiProcessorCount = 256;
  return hipSuccess;
}

namespace {
volatile unsigned char g_sink;
// Read and write back one byte at p + byte offset `at` (an access the sanitizer checks).
void touch(const void* p, size_t at) {
  if (p == nullptr) return;
  volatile unsigned char* q = (volatile unsigned char*)p + at;
  const unsigned char v = *q;
  *q = v;
  g_sink = v;
}
template <class T>
void extent(const T* p, int64_t n) {  // elements [0, n) are addressed
  if (p == nullptr || n <= 0) return;
  touch(p, 0);
  touch(p, (size_t)n * sizeof(T) - 1);
}
template <class T>
void rows(const T* p, int64_t nrows, int64_t ld, int64_t cols) {  // nrows x cols, stride ld
  if (p == nullptr || nrows <= 0 || cols <= 0) return;
  extent(p, (nrows - 1) * ld + cols);
}
int64_t g_launches = 0;
}  // namespace

extern "C" int64_t llp_stub_launches() { return g_launches; }

namespace llp {

alignas(256) static unsigned char g_scratch[SCRATCH_BYTES];

hipError_t probe_kernels() { return hipSuccess; }
hipError_t scratch_init(int device) { return device == 0 ? hipSuccess : hipErrorInvalidDevice; }
void* scratch_address(int device) { return device == 0 ? g_scratch : nullptr; }

// The device-side values the kernels read first (scored-row count) are unknown on the host:
// every extent below uses the worst case, all T rows scored.
hipError_t launch_layout(const LayoutArgs& a, hipStream_t) {
  ++g_launches;
  extent(a.mask, a.T);
  extent(a.targets, a.T);
  if (a.cu_seqlens) extent(a.cu_seqlens, (int64_t)a.num_seqs + 1);
  extent(a.count, 1 + (layout_blocks(a.T) > 1 ? layout_blocks(a.T) : 0));
  extent(a.scored, a.T);
  extent(a.pos, a.T);
  extent(a.tloc, a.T);
  extent(a.out_t, a.T); extent(a.out_f, a.T); extent(a.out_l, a.T);
  extent(a.out_e, a.T); extent(a.out_p, a.T);
  extent(a.qctr, a.nqctr);
  extent(a.status, 1);
  return hipSuccess;
}
hipError_t launch_fwd(const FwdArgs& a, hipStream_t) {
  ++g_launches;
  if (a.n_real > 0) rows(a.W, a.n_real, a.ldw, a.H);
  const int64_t Tc = (int64_t)a.ntb * 256;
  if (a.bias) extent((const unsigned char*)a.bias, a.n_real * (a.bias_f32 ? 4 : 2));
  for (const float* p : {a.pm, a.ps, a.pq}) extent(p, (int64_t)a.nvt * a.pstride);
  extent(a.tz, Tc);
  extent(a.scored, Tc);
  extent(a.tloc, Tc);
  extent(a.qctr, QCTR_INTS);
  return a.pstride >= Tc ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_combine(const CombineArgs& a, int64_t T_cap, hipStream_t) {
  ++g_launches;
  for (const float* p : {a.pm, a.ps, a.pq}) extent(p, (int64_t)a.nvt * a.pstride);
  extent(a.tz, T_cap);
  return hipSuccess;
}
hipError_t launch_merge(const MergeArgs& a, hipStream_t) {
  ++g_launches;
  for (int r = 0; r < a.world; ++r) {
    extent(a.tl[r], a.T); extent(a.flag[r], a.T); extent(a.lse[r], a.T); extent(a.ent[r], a.T);
  }
  extent(a.mask, a.T);
  extent(a.out_p, a.T); extent(a.out_l, a.T); extent(a.out_e, a.T);
  return hipSuccess;
}
hipError_t launch_topp(const ToppArgs& a, hipStream_t) {
  ++g_launches;
  if (a.n_real > 0)
    rows((const unsigned char*)a.logits, a.T, a.lstride * (a.bf16 ? 2 : 4), a.n_real * (a.bf16 ? 2 : 4));
  rows(a.ids, a.T, a.ids_stride, a.K);
  extent(a.targets, a.T); extent(a.mask, a.T);
  extent(a.out_t, a.T); extent(a.out_f, a.T); extent(a.out_l, a.T); extent(a.out_p, a.T);
  return hipSuccess;
}
hipError_t launch_grad(const GradArgs& a, hipStream_t) {
  ++g_launches;
  const int64_t Tc = (int64_t)a.ntb * 256;
  if (a.n_real > 0) rows(a.W, a.n_real, a.ldw, a.H);
  // G rows up to the next whole K step past the count, every vocabulary tile's columns.
  rows(a.G, Tc, a.ldg, (int64_t)a.nvt * 256);
  extent(a.qctr, QCTR_INTS);
  if (a.dbp) rows(a.dbp, a.ntb, a.ldg, (int64_t)a.nvt * 256);
  return a.ldg >= (int64_t)a.nvt * 256 ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_dh(const DhArgs& a, hipStream_t) {
  ++g_launches;
  rows(a.G, (int64_t)a.ntm * 256, a.ldg, (int64_t)a.nks * KSTEP);
  if (a.n_real > 0) rows(a.W, a.n_real, a.ldw, a.H);
  extent(a.P, (int64_t)a.nsplit * a.pstride * a.H);
  extent(a.qctr, QCTR_INTS);
  return hipSuccess;
}
hipError_t launch_dh_reduce(const DhReduceArgs& a, hipStream_t) {
  ++g_launches;
  extent(a.pos, a.T);
  if (a.nsplit > 0) extent(a.P, (int64_t)a.nsplit * a.pstride * a.H);
  rows(a.dH, a.T, a.ldd, a.H);
  return hipSuccess;
}
hipError_t launch_dw(const DwArgs& a, hipStream_t) {
  ++g_launches;
  rows(a.hgT, a.H, a.ldk, a.ldk);
  rows(a.G, a.ldk, a.ldg, (int64_t)a.ntm * 256);
  rows(a.dW, a.n_real, a.lddw, a.H);
  extent(a.qctr, QCTR_INTS);
  return hipSuccess;
}
hipError_t launch_transpose(const TransposeArgs& a, int64_t nrows, hipStream_t) {
  ++g_launches;
  rows(a.out, a.cols, a.ldo, nrows);
  extent(a.idx, nrows);
  return hipSuccess;
}
hipError_t launch_dbias(const DbArgs& a, hipStream_t) {
  ++g_launches;
  extent(a.db, a.n_real);
  if (a.n_real > 0) extent(a.dbp, a.n_real);   // at least the first token block's row
  return hipSuccess;
}
hipError_t launch_zero_rows(const ZeroArgs& a, hipStream_t) {
  ++g_launches;
  if (a.r1 > a.r0) rows(a.p + a.r0 * a.ld, a.r1 - a.r0, a.ld, a.cols);
  return hipSuccess;
}
hipError_t launch_logits(const LogitsArgs& a, hipStream_t) {
  ++g_launches;
  if (a.n_real > 0)
    rows((const unsigned char*)a.logits, a.T, a.ld * (a.bf16 ? 2 : 4), a.n_real * (a.bf16 ? 2 : 4));
  extent(a.targets, a.T); extent(a.mask, a.T);
  extent(a.out_t, a.T); extent(a.out_f, a.T); extent(a.out_l, a.T); extent(a.out_e, a.T);
  extent(a.out_p, a.T);
  return hipSuccess;
}
hipError_t launch_keep(const KeepArgs& a, hipStream_t) {
  ++g_launches;
  if (a.n_real > 0) {
    rows((const unsigned char*)a.logits, a.T, a.lstride * (a.bf16 ? 2 : 4), a.n_real * (a.bf16 ? 2 : 4));
    rows(a.keep, a.T, a.kstride, a.n_real);
  }
  extent(a.targets, a.T); extent(a.mask, a.T);
  extent(a.out_t, a.T); extent(a.out_f, a.T); extent(a.out_l, a.T); extent(a.out_p, a.T);
  return hipSuccess;
}

}  // namespace llp
