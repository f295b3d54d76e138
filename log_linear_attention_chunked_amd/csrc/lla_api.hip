// lla_api.hip — C ABI of the log-linear Mamba-2 forward pass: argument validation, plan
// (chunk, sweep, workspace layout), and the stream-ordered launch sequence: the forward kernel,
// preceded by a fill of the ticket counter and node flags only when the library allocates the
// workspace itself.
// The contract is documented in include/loglinear_attn.h.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <string.h>

#include "loglinear_attn.h"
#include "lla_dispatch.hpp"
#include "lla_host.hpp"
#include "lla_kernels.hpp"

namespace lla {

const KernelSet* kernel_set(int dtype, int C, int DK, int DV) {
  if (dtype == LLA_DTYPE_BF16) {
    switch (C) {
      case 16: return kernels_bf16_c16(DK, DV);
      case 32: return kernels_bf16_c32(DK, DV);
      case 64: return kernels_bf16_c64(DK, DV);
      case 128: return kernels_bf16_c128(DK, DV);
    }
  } else if (dtype == LLA_DTYPE_F32) {
    switch (C) {
      case 16: return kernels_f32_c16(DK, DV);
      case 32: return kernels_f32_c32(DK, DV);
      case 64: return kernels_f32_c64(DK, DV);
      case 128: return kernels_f32_c128(DK, DV);
    }
  }
  return nullptr;
}

}  // namespace lla

namespace lla {

// Zero-fills the ticket counter and the node flags of a freshly allocated workspace (a fill
// kernel rather than a memset so that the sequence stays safe to capture in a graph).
__global__ void lla_reset_kernel(int* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

}  // namespace lla

namespace {

using lla::KernelSet;
using lla::Params;

inline bool supported_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
inline int bit_len(unsigned x) { int n = 0; while (x) { ++n; x >>= 1; } return n; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kSpinLimit = 1 << 20;        // polls of a node flag (each ~1 us) before giving up
using lla::kLdsPerCU;
constexpr long kMinWorkgroups = 128;       // below this, prefer one chunk per workgroup

struct Plan {
  int C, R, m, nchunks, nsweep, ns, L, esize, nw;
  long BH;
  size_t ws_bytes, off_sync, off_gnode, off_nodeT, n_sync;
  int smem;
};

// Default chunk size and sweep length, from forward-kernel times measured on MI355X over every
// chunk/sweep that fits (bench.py --tune) for 17 shapes (B·H from 2 to 64, T from 256 to 131072,
// d from 16 to 128, both dtypes):
//   * what matters is the tokens a workgroup holds, C·R: 128 (chunk 64 with sweep 2, or chunk 128
//     with sweep 1) was fastest or within 1.5% of it at every bfloat16 shape with enough
//     workgroups, for every head size (d = 16: 22.9 µs against 44.7 at chunk 16, sweep 2);
//   * chunk 128 beat chunk 64 with sweep 2 by 1-3% at dk = dv = 128 and T >= 65536 (1 x 8 x 65536:
//     339 vs 347 µs; 1 x 32 x 65536: 1190 vs 1230; 1 x 2 x 131072: 221 vs 223), and tied below;
//   * sweep 2 lost once fewer than 128 workgroups were left (1 x 2 x 2048: 15.4 vs 14.7 µs) and won
//     above (2 x 8 x 2048, 256 workgroups: 17.6 vs 21.6);
//   * float32 lost at sweep 2 (4 x 16 x 8192, d = 64: 417 vs 372 µs: the images of two chunks leave
//     one workgroup of 4 waves per compute unit), and chunk 32 led at d = 16 (10.8 vs 11.8 µs at
//     chunk 16).
int default_chunk(int dk, int dv, int T, int esize) {
  if (esize == 4) return (dk <= 16 && dv <= 16) ? 32 : 64;
  if (dk == 128 && dv == 128 && T >= 65536) return 128;
  return 64;
}

int smem_bytes(int esize, int C, int dk, int dv, int R) {
  return lla::smem_layout(esize, C, dk, dv, R).total;
}

int default_sweep(long BH, int T, int C, int dk, int dv, int esize) {
  const int nchunks = (T + C - 1) / C;
  if (nchunks <= 1 || esize == 4) return 1;
  if (smem_bytes(esize, C, dk, dv, 2) > kLdsPerCU) return 1;
  return BH * ((nchunks + 1) / 2) >= kMinWorkgroups ? 2 : 1;
}

// Host-only part of the plan: sizes and layout; no device calls.
int make_plan(int B, int H, int T, int dk, int dv, int chunk, int sweep, int dtype, Plan& pl) {
  if (dtype != LLA_DTYPE_BF16 && dtype != LLA_DTYPE_F32) return LLA_ERR_INVALID_ARG;
  if (B < 0 || H < 0 || T < 0) return LLA_ERR_INVALID_ARG;
  if (!supported_dim(dk) || !supported_dim(dv)) return LLA_ERR_UNSUPPORTED;
  if (chunk != 0 && !supported_dim(chunk)) return LLA_ERR_UNSUPPORTED;
  if (sweep != 0 && sweep != 1 && sweep != 2) return LLA_ERR_UNSUPPORTED;
  const int C = chunk ? chunk : default_chunk(dk, dv, T, dtype == LLA_DTYPE_F32 ? 4 : 2);
  const long BH = (long)B * H;
  if (BH > 65535) return LLA_ERR_UNSUPPORTED;
  pl.C = C;
  pl.BH = BH;
  pl.L = T > 0 ? bit_len((unsigned)(T - 1)) + 1 : 0;
  if (pl.L > lla::kLamCap) return LLA_ERR_UNSUPPORTED;
  pl.esize = dtype == LLA_DTYPE_BF16 ? 2 : 4;
  pl.nw = dv / 16;
  pl.nchunks = (T + C - 1) / C;
  pl.R = sweep ? sweep : default_sweep(BH, T, C, dk, dv, pl.esize);
  pl.m = bit_len((unsigned)pl.R) - 1;
  pl.nsweep = pl.nchunks > 0 ? (pl.nchunks + pl.R - 1) / pl.R : 0;
  pl.ns = pl.nsweep > 1 ? pl.nsweep - 1 : 0;
  if ((long)pl.nsweep * BH > 0x7fffffffL) return LLA_ERR_UNSUPPORTED;   // one workgroup per sweep
  const size_t nodes = (size_t)BH * pl.ns * pl.nw;      // (head, node, wave) records
  size_t off = 0;
  pl.n_sync = lla::kFlagBase + nodes;
  pl.off_sync = off;   off = align256(off + pl.n_sync * 4);
  pl.off_gnode = off;  off = align256(off + nodes * 4);
  pl.off_nodeT = off;  off = align256(off + nodes * ((dk + 31) / 32) * 64 * 8 * pl.esize);
  pl.ws_bytes = pl.ns > 0 ? off : 0;
  pl.smem = smem_bytes(pl.esize, C, dk, dv, pl.R);
  // the sweep's images must fit one compute unit's shared memory (float32 at large chunk and
  // head sizes does not)
  if (pl.smem > kLdsPerCU) return LLA_ERR_UNSUPPORTED;
  return LLA_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

int validate_pointers(const lla_fwd_args& a, const Plan& pl) {
  if (!a.q || !a.k || !a.v || !a.log_a || !a.lambda || !a.out) return LLA_ERR_INVALID_ARG;
  const size_t es = (size_t)pl.esize;
  const size_t nt = (size_t)pl.BH * a.T;
  if (a.lambda_bf16 != 0 && a.lambda_bf16 != 1) return LLA_ERR_INVALID_ARG;
  const size_t lsz = a.lambda_bf16 ? 2 : 4;
  const size_t nq = nt * a.dk * es, nv = nt * a.dv * es, nla = nt * 4, nlam = nt * pl.L * lsz;
  if (((uintptr_t)a.q | (uintptr_t)a.k | (uintptr_t)a.v | (uintptr_t)a.out) & 15) return LLA_ERR_INVALID_ARG;
  if (((uintptr_t)a.log_a & 3) || ((uintptr_t)a.lambda & (lsz - 1))) return LLA_ERR_INVALID_ARG;
  if (overlaps(a.out, nv, a.q, nq) || overlaps(a.out, nv, a.k, nq) || overlaps(a.out, nv, a.v, nv) ||
      overlaps(a.out, nv, a.log_a, nla) || overlaps(a.out, nv, a.lambda, nlam))
    return LLA_ERR_INVALID_ARG;
  return LLA_OK;
}

hipError_t set_smem(const void* fn, int bytes) {
  return bytes > 65536 ? hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes)
                       : hipSuccess;
}

// packed variable-length batch: N sequences of vH heads along T_packed rows
struct Varlen {
  const int* cu_seqlens;
  int vN, vH, T_packed;
  int tickets;      // workgroups that have a sweep (from a host copy of cu_seqlens), or 0
};

int launch(const lla_fwd_args& a, const Plan& pl, void* ws, bool fresh_ws, hipStream_t stream,
           const Varlen* vl = nullptr) {
  const KernelSet* ks = lla::kernel_set(a.dtype, pl.C, a.dk, a.dv);
  if (!ks) return LLA_ERR_UNSUPPORTED;

  int dev = 0, max_smem = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LLA_ERR_HIP;
  if (hipDeviceGetAttribute(&max_smem, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    return LLA_ERR_HIP;
  if (pl.smem > max_smem) return LLA_ERR_UNSUPPORTED;

  Params p;
  memset(&p, 0, sizeof(p));
  p.q = a.q; p.k = a.k; p.v = a.v; p.log_a = a.log_a; p.lam = a.lambda; p.out = a.out;
  p.lam_bf16 = a.lambda_bf16;
  p.BH = (int)pl.BH; p.T = a.T; p.L = pl.L;
  p.nchunks = pl.nchunks; p.sweep = pl.R; p.m = pl.m; p.nsweep = pl.nsweep;
  if (ws) {
    p.sync = reinterpret_cast<int*>((char*)ws + pl.off_sync);
    p.gnode = reinterpret_cast<float*>((char*)ws + pl.off_gnode);
    p.nodeT = (char*)ws + pl.off_nodeT;
  }
  p.spin_limit = kSpinLimit;
  if (vl) {
    p.T = vl->T_packed;
    p.cu_seqlens = vl->cu_seqlens;
    p.vN = vl->vN;
    p.vH = vl->vH;
    p.vtotal = vl->tickets;
  }
  void* args[] = {&p};
  auto mark = [&](int i) {
    return a.stage_events[i] ? hipEventRecord(reinterpret_cast<hipEvent_t>(a.stage_events[i]), stream)
                             : hipSuccess;
  };

  if (mark(0) != hipSuccess) return LLA_ERR_HIP;
  if (pl.ns > 0 && fresh_ws) {
    const int n = (int)pl.n_sync;
    const int blocks = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
    hipLaunchKernelGGL(lla::lla_reset_kernel, dim3(blocks), dim3(256), 0, stream, p.sync, n);
    if (hipGetLastError() != hipSuccess) return LLA_ERR_HIP;
  }
  if (mark(1) != hipSuccess) return LLA_ERR_HIP;
  const void* fn = vl ? ks->fwd_varlen[pl.R - 1] : ks->fwd[pl.R - 1];
  if (set_smem(fn, pl.smem) != hipSuccess) return LLA_ERR_HIP;
  const unsigned grid = (unsigned)(vl && vl->tickets ? vl->tickets : pl.nsweep * pl.BH);
  if (hipLaunchKernel(fn, dim3(grid), dim3(64 * pl.nw), args, pl.smem, stream) != hipSuccess)
    return LLA_ERR_HIP;
  if (mark(2) != hipSuccess) return LLA_ERR_HIP;
  return LLA_OK;
}

int run_forward(const lla_fwd_args& a, const Plan& pl, hipStream_t stream, const Varlen* vl) {
  void* ws = a.workspace;
  bool owned = false;
  if (pl.ws_bytes > 0) {
    if (ws) {
      if (a.workspace_bytes < pl.ws_bytes) return LLA_ERR_WORKSPACE;
      if ((uintptr_t)ws & 255) return LLA_ERR_INVALID_ARG;
    } else {
      if (lla::workspace_alloc(&ws, pl.ws_bytes, stream) != hipSuccess) return LLA_ERR_NO_MEMORY;
      owned = true;
    }
  }
  int st = launch(a, pl, ws, owned, stream, vl);
  if (owned && hipFreeAsync(ws, stream) != hipSuccess && st == LLA_OK) st = LLA_ERR_HIP;
  return st;
}

int forward_varlen(const lla_fwd_varlen_args& v, hipStream_t stream) {
  if (v.N < 0 || v.H < 0 || v.total_T < 0 || v.max_T < 0) return LLA_ERR_INVALID_ARG;
  if (v.dtype != LLA_DTYPE_BF16 && v.dtype != LLA_DTYPE_F32) return LLA_ERR_INVALID_ARG;
  if (v.max_T > v.total_T) return LLA_ERR_INVALID_ARG;
  // the plan of N x H heads of the longest length: chunk, sweep, grid and workspace
  Plan pl;
  int st = make_plan(v.N, v.H, v.max_T, v.dk, v.dv, v.chunk, v.sweep, v.dtype, pl);
  if (st != LLA_OK) return st;
  if (pl.BH == 0 || v.max_T == 0) return LLA_OK;
  // tensors are [H, total_T, .]; lambda has L = num_levels(max_T) levels per row
  lla_fwd_args a;
  memset(&a, 0, sizeof(a));
  a.q = v.q; a.k = v.k; a.v = v.v; a.log_a = v.log_a; a.lambda = v.lambda; a.out = v.out;
  a.lambda_bf16 = v.lambda_bf16;
  a.B = 1; a.H = v.H; a.T = v.total_T; a.dk = v.dk; a.dv = v.dv; a.dtype = v.dtype;
  a.workspace = v.workspace; a.workspace_bytes = v.workspace_bytes;
  Plan pp = pl;
  pp.BH = v.H;                         // pointer extents: H heads of total_T rows
  st = validate_pointers(a, pp);
  if (st != LLA_OK) return st;
  if (!v.cu_seqlens || ((uintptr_t)v.cu_seqlens & 3)) return LLA_ERR_INVALID_ARG;
  Varlen vl{v.cu_seqlens, v.N, v.H, v.total_T, 0};
  if (v.cu_seqlens_host) {
    // the workgroups that have a sweep, with the kernel's clamping of each sequence
    long long sweeps = 0;
    const long long span = (long long)pl.nchunks * pl.C;
    for (int n = 0; n < v.N; ++n) {
      const long long s0 = std::min<long long>(std::max(v.cu_seqlens_host[n], 0), v.total_T);
      const long long s1 = std::min<long long>(std::max<long long>(v.cu_seqlens_host[n + 1], s0),
                                               std::min<long long>(s0 + span, v.total_T));
      const long long nch = (s1 - s0 + pl.C - 1) / pl.C;
      sweeps += (nch + pl.R - 1) / pl.R;
    }
    if (sweeps == 0) return LLA_OK;
    vl.tickets = (int)(sweeps * v.H);
  }
  return run_forward(a, pl, stream, &vl);
}

int forward(const lla_fwd_args& a, hipStream_t stream) {
  Plan pl;
  int st = make_plan(a.B, a.H, a.T, a.dk, a.dv, a.chunk, a.sweep, a.dtype, pl);
  if (st != LLA_OK) return st;
  if (pl.BH == 0 || a.T == 0) return LLA_OK;
  st = validate_pointers(a, pl);
  if (st != LLA_OK) return st;
  return run_forward(a, pl, stream, nullptr);
}

// ---- the entry point that allocates nothing: a fixed scratch array per device ----------------
//
// The forward kernel's workspace (ticket counter, node flags, node decays and node records) lives
// in this static device array instead. Each device that runs the entry point holds its own copy
// until the process ends. Its name is a host-side stand-in in host code: the device address is
// taken once per device with hipGetSymbolAddress and only that address is ever passed on.
constexpr size_t kScratchBytes = (size_t)64 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];          // device address of `scratch` on each device, once known

// The scratch of the current device: its address is looked up on the first call on the device,
// and the whole array is zero-filled then by a fill kernel on `stream` (the ticket counter and
// flags must start at zero once; every call leaves them ready for the next one).
int device_scratch(hipStream_t stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return LLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return LLA_ERR_HIP;
    const int n = (int)(kScratchBytes / 4);
    hipLaunchKernelGGL(lla::lla_reset_kernel, dim3(1024), dim3(256), 0, stream, static_cast<int*>(ptr), n);
    if (hipGetLastError() != hipSuccess) return LLA_ERR_HIP;
    scratch_ptr[dev] = ptr;
  }
  *out = scratch_ptr[dev];
  return LLA_OK;
}

int forward_noalloc(const lla_fwd_args& a, hipStream_t stream) {
  if (a.workspace || a.workspace_bytes) return LLA_ERR_INVALID_ARG;   // the scratch replaces it
  Plan pl;
  int st = make_plan(a.B, a.H, a.T, a.dk, a.dv, a.chunk, a.sweep, a.dtype, pl);
  if (st != LLA_OK) return st;
  if (pl.ws_bytes > kScratchBytes) return LLA_ERR_SCRATCH_LIMIT;
  if (pl.BH == 0 || a.T == 0) return LLA_OK;
  st = validate_pointers(a, pl);
  if (st != LLA_OK) return st;
  void* ws = nullptr;
  if (pl.ws_bytes > 0) {
    st = device_scratch(stream, &ws);
    if (st != LLA_OK) return st;
  }
  return launch(a, pl, ws, false, stream, nullptr);
}

}  // namespace

extern "C" {

int loglinear_attn_fwd_ex(const lla_fwd_args* args, lla_stream_t stream) {
  if (!args) return LLA_ERR_INVALID_ARG;
  return forward(*args, reinterpret_cast<hipStream_t>(stream));
}

int loglinear_attn_fwd_noalloc(const lla_fwd_args* args, lla_stream_t stream) {
  if (!args) return LLA_ERR_INVALID_ARG;
  return forward_noalloc(*args, reinterpret_cast<hipStream_t>(stream));
}

size_t loglinear_attn_noalloc_scratch_bytes(void) { return kScratchBytes; }

int loglinear_attn_fwd_varlen(const lla_fwd_varlen_args* args, lla_stream_t stream) {
  if (!args) return LLA_ERR_INVALID_ARG;
  return forward_varlen(*args, reinterpret_cast<hipStream_t>(stream));
}

int loglinear_attn_fwd(const void* q, const void* k, const void* v, const float* log_a,
                       const float* lambda, void* out, int B, int H, int T, int dk, int dv,
                       lla_stream_t stream) {
  lla_fwd_args a;
  memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.v = v; a.log_a = log_a; a.lambda = lambda; a.out = out;
  a.B = B; a.H = H; a.T = T; a.dk = dk; a.dv = dv; a.dtype = LLA_DTYPE_BF16;
  return forward(a, reinterpret_cast<hipStream_t>(stream));
}

int loglinear_attn_fwd_f32(const float* q, const float* k, const float* v, const float* log_a,
                           const float* lambda, float* out, int B, int H, int T, int dk, int dv,
                           lla_stream_t stream) {
  lla_fwd_args a;
  memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.v = v; a.log_a = log_a; a.lambda = lambda; a.out = out;
  a.B = B; a.H = H; a.T = T; a.dk = dk; a.dv = dv; a.dtype = LLA_DTYPE_F32;
  return forward(a, reinterpret_cast<hipStream_t>(stream));
}

size_t loglinear_attn_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int sweep,
                                      int dtype) {
  Plan pl;
  if (make_plan(B, H, T, dk, dv, chunk, sweep, dtype, pl) != LLA_OK) return 0;
  return pl.ws_bytes;
}

int loglinear_attn_num_levels(int T) { return T > 0 ? bit_len((unsigned)(T - 1)) + 1 : 0; }

int loglinear_attn_default_chunk(int dk, int dv, int T, int dtype) {
  if (!supported_dim(dk) || !supported_dim(dv) || T < 0) return 0;
  if (dtype != LLA_DTYPE_BF16 && dtype != LLA_DTYPE_F32) return 0;
  return default_chunk(dk, dv, T, dtype == LLA_DTYPE_F32 ? 4 : 2);
}

int loglinear_attn_default_sweep(int B, int H, int T, int dk, int dv, int chunk, int dtype) {
  if (B < 0 || H < 0 || T < 0) return 0;
  if (dtype != LLA_DTYPE_BF16 && dtype != LLA_DTYPE_F32) return 0;
  const int C = chunk ? chunk : default_chunk(dk, dv, T, dtype == LLA_DTYPE_F32 ? 4 : 2);
  if (!supported_dim(C) || !supported_dim(dk) || !supported_dim(dv)) return 0;
  return default_sweep((long)B * H, T, C, dk, dv, dtype == LLA_DTYPE_F32 ? 4 : 2);
}

const char* loglinear_attn_status_string(int status) {
  switch (status) {
    case LLA_OK: return "ok";
    case LLA_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, negative size, aliasing output)";
    case LLA_ERR_UNSUPPORTED: return "unsupported shape (dk, dv or chunk outside {16,32,64,128}, sweep, level count or shared memory)";
    case LLA_ERR_HIP: return "HIP runtime call or kernel launch failed";
    case LLA_ERR_NO_MEMORY: return "workspace allocation failed";
    case LLA_ERR_WORKSPACE: return "caller workspace too small";
    case LLA_ERR_SCRATCH_LIMIT: return "the call needs more workspace than the fixed scratch of loglinear_attn_fwd_noalloc";
    default: return "unknown status";
  }
}

}  // extern "C"
