// lla_gdn_api.hip — C ABI of the log-linear Gated DeltaNet forward pass: argument validation,
// plan (chunk, tree slots, workspace layout) and the stream-ordered launches gdn_chunk ->
// gdn_upsweep (one per tree level) -> gdn_query. The contract is documented in
// include/loglinear_attn.h.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "lla_gdn.hpp"
#include "lla_host.hpp"
#include "loglinear_attn.h"

namespace {

using lla::gdn::GdnKernels;
using lla::gdn::GdnParams;

inline bool supported_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
inline int bit_len(unsigned x) { int n = 0; while (x) { ++n; x >>= 1; } return n; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

const GdnKernels* gdn_kernels(int dtype, int C, int dk, int dv) {
  using namespace lla::gdn;
  if (dtype == LLA_DTYPE_BF16)
    return C == 16 ? kernels_bf16_c16(dk, dv) : C == 32 ? kernels_bf16_c32(dk, dv) : C == 64 ? kernels_bf16_c64(dk, dv) : nullptr;
  if (dtype == LLA_DTYPE_F32)
    return C == 16 ? kernels_f32_c16(dk, dv) : C == 32 ? kernels_f32_c32(dk, dv) : C == 64 ? kernels_f32_c64(dk, dv) : nullptr;
  return nullptr;
}

// the up-sweep kernel depends on (dk, dv) only
template <int DK, bool WHOLE>
const void* upsweep_for_dv(int dv) {
  switch (dv) {
    case 16: return reinterpret_cast<const void*>(&lla::gdn::gdn_upsweep_kernel<DK, 16, WHOLE>);
    case 32: return reinterpret_cast<const void*>(&lla::gdn::gdn_upsweep_kernel<DK, 32, WHOLE>);
    case 64: return reinterpret_cast<const void*>(&lla::gdn::gdn_upsweep_kernel<DK, 64, WHOLE>);
    case 128: return reinterpret_cast<const void*>(&lla::gdn::gdn_upsweep_kernel<DK, 128, WHOLE>);
  }
  return nullptr;
}
// whole rows only for dk <= 64 (a 128 x 128 transition fills 66 KB of shared memory by itself)
const void* upsweep_kernel(int dk, int dv, bool whole) {
  switch (dk) {
    case 16: return whole ? upsweep_for_dv<16, true>(dv) : upsweep_for_dv<16, false>(dv);
    case 32: return whole ? upsweep_for_dv<32, true>(dv) : upsweep_for_dv<32, false>(dv);
    case 64: return whole ? upsweep_for_dv<64, true>(dv) : upsweep_for_dv<64, false>(dv);
    case 128: return whole ? nullptr : upsweep_for_dv<128, false>(dv);
  }
  return nullptr;
}
// a level's nodes times heads from which one workgroup per node beats 16-column panels (at
// fewer, the panels' extra workgroups fill the device better)
constexpr long kUpWholeMin = 1024;
// two levels in one launch (dk <= 64): the fold of four grandchildren per workgroup, its
// products in split bf16 for bfloat16 inputs with dk >= 32 (as the query kernel's)
template <int DK, bool BF3>
const void* upsweep2_for_dv(int dv) {
  switch (dv) {
    case 16: return reinterpret_cast<const void*>(&lla::gdn::gdn_upsweep2_kernel<DK, 16, BF3>);
    case 32: return reinterpret_cast<const void*>(&lla::gdn::gdn_upsweep2_kernel<DK, 32, BF3>);
    case 64: return reinterpret_cast<const void*>(&lla::gdn::gdn_upsweep2_kernel<DK, 64, BF3>);
    case 128: return reinterpret_cast<const void*>(&lla::gdn::gdn_upsweep2_kernel<DK, 128, BF3>);
  }
  return nullptr;
}
const void* upsweep2_kernel(int dk, int dv, bool bf3) {
  switch (dk) {
    case 16: return upsweep2_for_dv<16, false>(dv);
    case 32: return bf3 ? upsweep2_for_dv<32, true>(dv) : upsweep2_for_dv<32, false>(dv);
    case 64: return bf3 ? upsweep2_for_dv<64, true>(dv) : upsweep2_for_dv<64, false>(dv);
  }
  return nullptr;
}
inline bool up2_bf3(int dtype, int dk) { return dtype == LLA_DTYPE_BF16 && dk >= 32; }


bool fits(int C, int dk, int dv) {
  using namespace lla::gdn;
  return chunk_smem_bytes(C, dk, dv) <= lla::kLdsPerCU && query_smem_bytes(C, dk, dv) <= lla::kLdsPerCU;
}

// chunk 32 where it fits (every supported head size), else 16. Measured on MI355X (time per
// call, chunks 64 / 32 / 16): 2.12 / 1.86 / 2.46 ms at B=4, H=16, T=8192, d=64 (bf16 and fp32
// alike); 0.40 / 0.27 / 0.32 ms at d=16 and 0.95 / 0.58 / 0.71 ms at d=32 there; 0.146 / 0.143 /
// 0.188 ms at B=2, H=8, T=2048, d=64; 2.26 / 1.95 / 2.59 ms at B=1, H=16, T=32768, d=64;
// - / 1.33 / 1.96 ms at B=1, H=8, T=8192, d=128. At chunk 64 one workgroup of the chunk kernel
// fills a compute unit's shared memory (140 KB at d=64); at 32 two fit, and the chunk kernel's
// C^2 and C*d^2 work per chunk shrinks faster than the longer tree grows
int default_chunk(int dk, int dv) {
  for (int C : {32, 16})
    if (fits(C, dk, dv)) return C;
  return 0;
}

struct GdnPlan {
  int C, N, L, esize, nslot, top;   // top: highest tree level built (0 = leaves only)
  long BH;
  size_t off_oi, off_x0, off_node, off_phi, ws_bytes;
};

int make_plan(int B, int H, int T, int dk, int dv, int chunk, int dtype, GdnPlan& pl) {
  if (dtype != LLA_DTYPE_BF16 && dtype != LLA_DTYPE_F32) return LLA_ERR_INVALID_ARG;
  if (B < 0 || H < 0 || T < 0) return LLA_ERR_INVALID_ARG;
  if (!supported_dim(dk) || !supported_dim(dv)) return LLA_ERR_UNSUPPORTED;
  if (chunk != 0 && chunk != 16 && chunk != 32 && chunk != 64) return LLA_ERR_UNSUPPORTED;
  const int C = chunk ? chunk : default_chunk(dk, dv);
  if (C == 0 || !fits(C, dk, dv)) return LLA_ERR_UNSUPPORTED;
  const long BH = (long)B * H;
  if (BH > 65535) return LLA_ERR_UNSUPPORTED;
  pl.C = C;
  pl.BH = BH;
  pl.L = T > 0 ? bit_len((unsigned)(T - 1)) + 1 : 0;
  if (pl.L > lla::gdn::kLamCapG) return LLA_ERR_UNSUPPORTED;
  pl.esize = dtype == LLA_DTYPE_BF16 ? 2 : 4;
  pl.N = (T + C - 1) / C;
  if ((long)pl.N * BH > 0x7fffffffL) return LLA_ERR_UNSUPPORTED;
  // the highest chunk bit any chunk index has: levels 1..top are built, node (j, m) for m < N >> j
  pl.top = pl.N > 1 ? bit_len((unsigned)(pl.N - 1)) - 1 : 0;
  pl.nslot = 0;
  for (int j = 0; j <= pl.top; ++j) pl.nslot += pl.N >> j;
  const size_t rows = (size_t)BH * pl.N * C;
  size_t off = 0;
  pl.off_oi = off;   off = align256(off + rows * dv * 4);
  pl.off_x0 = off;   off = align256(off + rows * dk * 4);
  pl.off_node = off; off = align256(off + (size_t)BH * pl.nslot * dk * dv * 4);
  pl.off_phi = off;  off = align256(off + (size_t)BH * pl.nslot * dk * dk * 4);
  pl.ws_bytes = off;
  return LLA_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

int validate(const lla_gdn_args& a, const GdnPlan& pl) {
  if (!a.q || !a.k || !a.v || !a.log_a || !a.beta || !a.lambda || !a.out) return LLA_ERR_INVALID_ARG;
  if (a.lambda_bf16 != 0 && a.lambda_bf16 != 1) return LLA_ERR_INVALID_ARG;
  const size_t es = (size_t)pl.esize, nt = (size_t)pl.BH * a.T, ls = a.lambda_bf16 ? 2 : 4;
  const size_t nq = nt * a.dk * es, nv = nt * a.dv * es, n4 = nt * 4, nl = nt * pl.L * ls;
  if (((uintptr_t)a.q | (uintptr_t)a.k | (uintptr_t)a.v | (uintptr_t)a.out) & 15) return LLA_ERR_INVALID_ARG;
  if (((uintptr_t)a.log_a | (uintptr_t)a.beta) & 3) return LLA_ERR_INVALID_ARG;
  if ((uintptr_t)a.lambda & (ls - 1)) return LLA_ERR_INVALID_ARG;
  if (overlaps(a.out, nv, a.q, nq) || overlaps(a.out, nv, a.k, nq) || overlaps(a.out, nv, a.v, nv) ||
      overlaps(a.out, nv, a.log_a, n4) || overlaps(a.out, nv, a.beta, n4) || overlaps(a.out, nv, a.lambda, nl))
    return LLA_ERR_INVALID_ARG;
  return LLA_OK;
}

hipError_t set_smem(const void* fn, int bytes) {
  return bytes > 65536 ? hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes)
                       : hipSuccess;
}

int launch(const lla_gdn_args& a, const GdnPlan& pl, void* ws, hipStream_t stream) {
  using namespace lla::gdn;
  const GdnKernels* ks = gdn_kernels(a.dtype, pl.C, a.dk, a.dv);
  const void* up = upsweep_kernel(a.dk, a.dv, false);
  const void* upw = upsweep_kernel(a.dk, a.dv, true);   // null at dk = 128
  const void* up2 = upsweep2_kernel(a.dk, a.dv, up2_bf3(a.dtype, a.dk));   // null at dk = 128
  if (!ks || !up) return LLA_ERR_UNSUPPORTED;
  GdnParams p;
  memset(&p, 0, sizeof(p));
  p.q = a.q; p.k = a.k; p.v = a.v; p.log_a = a.log_a; p.beta = a.beta; p.lam = a.lambda; p.out = a.out;
  p.lam_bf16 = a.lambda_bf16;
  p.BH = (int)pl.BH; p.T = a.T; p.L = pl.L; p.nchunks = pl.N; p.nslot = pl.nslot;
  p.oi = reinterpret_cast<float*>((char*)ws + pl.off_oi);
  p.x0 = reinterpret_cast<float*>((char*)ws + pl.off_x0);
  p.node = reinterpret_cast<float*>((char*)ws + pl.off_node);
  p.phi = reinterpret_cast<float*>((char*)ws + pl.off_phi);
  auto mark = [&](int i) {
    return a.stage_events[i] ? hipEventRecord(reinterpret_cast<hipEvent_t>(a.stage_events[i]), stream)
                             : hipSuccess;
  };
  const unsigned grid = (unsigned)(pl.N * pl.BH);
  const int sc = chunk_smem_bytes(pl.C, a.dk, a.dv, a.dtype == LLA_DTYPE_BF16);
  const int sq = query_smem_bytes(pl.C, a.dk, a.dv, a.dtype == LLA_DTYPE_BF16);
  const int su = up_smem_bytes(a.dk, a.dv, false), suw = up_smem_bytes(a.dk, a.dv, true);
  const int su2 = up2_smem_bytes(a.dk, a.dv, up2_bf3(a.dtype, a.dk));
  if (mark(0) != hipSuccess) return LLA_ERR_HIP;
  {
    void* args[] = {&p};
    if (set_smem(ks->chunk, sc) != hipSuccess) return LLA_ERR_HIP;
    if (hipLaunchKernel(ks->chunk, dim3(grid), dim3(kNT), args, sc, stream) != hipSuccess) return LLA_ERR_HIP;
  }
  if (mark(1) != hipSuccess) return LLA_ERR_HIP;
  if (set_smem(up, su) != hipSuccess) return LLA_ERR_HIP;
  if (upw && set_smem(upw, suw) != hipSuccess) return LLA_ERR_HIP;
  if (up2 && set_smem(up2, su2) != hipSuccess) return LLA_ERR_HIP;
  int off_prev = 0;   // first slot of level j - 1
  for (int j = 1; j <= pl.top;) {
    GdnParams pj = p;
    pj.level = j;
    pj.off_prev = off_prev;
    pj.off_cur = off_prev + (pl.N >> (j - 1));
    pj.off_next = pj.off_cur + (pl.N >> j);
    pj.ncur = pl.N >> j;
    void* args[] = {&pj};
    if (up2) {
      // for dk <= 64 every level goes through gdn_upsweep2 (its split-bf16 form reads and writes
      // the nodes as high and low parts, which no other up-sweep kernel reads): two levels at a
      // time, and a last odd level's even nodes on their own
      pj.two = j + 1 <= pl.top ? 1 : 0;
      const long nwg = pj.two ? (long)((pj.ncur >> 1) + (pj.ncur & 1)) * pl.BH : (long)((pj.ncur + 1) >> 1) * pl.BH;
      if (hipLaunchKernel(up2, dim3((unsigned)nwg), dim3(kNT), args, su2, stream) != hipSuccess) return LLA_ERR_HIP;
      off_prev = pj.two ? pj.off_next : pj.off_cur;
      j += pj.two ? 2 : 1;
      continue;
    }
    const bool whole = upw && (long)pj.ncur * pl.BH >= kUpWholeMin;
    const unsigned g = (unsigned)((long)pj.ncur * pl.BH * ((a.dv + a.dk) / up_panel(a.dk, a.dv, whole)));
    if (hipLaunchKernel(whole ? upw : up, dim3(g), dim3(kNT), args, whole ? suw : su, stream) != hipSuccess)
      return LLA_ERR_HIP;
    off_prev = pj.off_cur;
    j += 1;
  }
  if (mark(2) != hipSuccess) return LLA_ERR_HIP;
  {
    void* args[] = {&p};
    if (set_smem(ks->query, sq) != hipSuccess) return LLA_ERR_HIP;
    if (hipLaunchKernel(ks->query, dim3(grid), dim3(kNT), args, sq, stream) != hipSuccess) return LLA_ERR_HIP;
  }
  if (mark(3) != hipSuccess) return LLA_ERR_HIP;
  return LLA_OK;
}

int gdn_forward(const lla_gdn_args& a, hipStream_t stream) {
  GdnPlan pl;
  int st = make_plan(a.B, a.H, a.T, a.dk, a.dv, a.chunk, a.dtype, pl);
  if (st != LLA_OK) return st;
  if (pl.BH == 0 || a.T == 0) return LLA_OK;
  st = validate(a, pl);
  if (st != LLA_OK) return st;
  void* ws = a.workspace;
  bool owned = false;
  if (ws) {
    if (a.workspace_bytes < pl.ws_bytes) return LLA_ERR_WORKSPACE;
    if ((uintptr_t)ws & 255) return LLA_ERR_INVALID_ARG;
  } else {
    if (lla::workspace_alloc(&ws, pl.ws_bytes, stream) != hipSuccess) return LLA_ERR_NO_MEMORY;
    owned = true;
  }
  st = launch(a, pl, ws, stream);
  if (owned && hipFreeAsync(ws, stream) != hipSuccess && st == LLA_OK) st = LLA_ERR_HIP;
  return st;
}

}  // namespace

extern "C" {

int loglinear_attn_gdn_fwd(const lla_gdn_args* args, lla_stream_t stream) {
  if (!args) return LLA_ERR_INVALID_ARG;
  return gdn_forward(*args, reinterpret_cast<hipStream_t>(stream));
}

size_t loglinear_attn_gdn_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int dtype) {
  GdnPlan pl;
  if (make_plan(B, H, T, dk, dv, chunk, dtype, pl) != LLA_OK) return 0;
  return pl.ws_bytes;
}

int loglinear_attn_gdn_default_chunk(int dk, int dv, int dtype) {
  if (!supported_dim(dk) || !supported_dim(dv)) return 0;
  if (dtype != LLA_DTYPE_BF16 && dtype != LLA_DTYPE_F32) return 0;
  return default_chunk(dk, dv);
}

}  // extern "C"
