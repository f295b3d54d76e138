/*
 * loglinear_attn.h — C ABI of the MI355X (gfx950) log-linear Mamba-2 attention: the forward pass,
 * and further below its variable-length, decoding, prefill and backward entry points.
 *
 * Operation (per batch b and head h, every position t in [0, T)):
 *
 *   o_t = sum_{s <= t} lambda[t, l(t,s)] * prod_{r=s+1..t} a_r * (q_t . k_s) * v_s
 *   l(t, s) = bit_length(t XOR s)      (0-based positions; 0 when s == t)
 *   a_r     = exp(log_a[r])
 *
 * Sources ("Log-Linear Attention", arXiv 2506.04761, as explained on the study-notes
 * page dimensionstp.github.io/study-concept/log_linear_attention and the gist.science
 * summaries): the output is a lambda-weighted sum over Fenwick-tree levels of
 * per-level states (study notes, sections 2-2 and 3-3); the prefix is split into
 * power-of-two buckets (section 3-2); the parallel form is (QK^T * M)V with
 * M = M^S * M^H, the Mamba-2 decay mask times the hierarchical mask (sections 3-4,
 * 3-5); it is evaluated chunkwise, a dense masked block inside each chunk and
 * O(log(T/C)) state passes between chunks (gist.science zh technical summary,
 * section 2.3).
 *
 * Layout: every tensor is a dense row-major array in [B, H, T, ...] order:
 *   q, k   [B, H, T, dk]     v, out  [B, H, T, dv]
 *   log_a  [B, H, T]         lambda  [B, H, T, L],  L = loglinear_attn_num_levels(T)
 * q, k, v and out are bfloat16 in loglinear_attn_fwd and float32 in
 * loglinear_attn_fwd_f32; log_a and lambda are always float32. All accumulation is
 * float32. Pointers are device pointers (HIP device memory of the current device);
 * the caller owns every buffer. Inputs are read only; out is fully overwritten.
 *
 * Preconditions that are documented but not checked: log_a finite and <= 0,
 * lambda finite and >= 0 (the arithmetic does not depend on either sign, but
 * decay factors above 1 can overflow), q/k/v finite.
 *
 * Supported: B, H, T >= 0 (any product that is 0 is a no-op); B*H <= 65535;
 * dk, dv in {16, 32, 64, 128}; chunk in {16, 32, 64, 128}; any T up to 2^23
 * (L <= 24; a ragged last chunk is masked), provided the chunks one workgroup holds fit the
 * 160 KB of shared memory of a compute unit:
 *   R * (C*(2*dk + dv)*e + 112*C + 16 + (C/16)*ceil(C/32)*512*e) + 272 <= 163840
 * (R chunks per workgroup, e = element bytes). bfloat16 always fits at R = 1; float32 with
 * chunk 128 and 2*dk + dv >= 192 fits at no R, and R = 2 does not fit for bfloat16 at chunk
 * 128 with dk >= 64 or dv = 128, nor for float32 at chunk 128 or at chunk 64 with dk = 128 or
 * dk = 64, dv = 128. Combinations that do not fit return LLA_ERR_UNSUPPORTED from the host-side
 * checks, before any device call (and loglinear_attn_workspace_bytes returns 0 for them); the
 * library's default chunk and sweep always fit. Output is bitwise deterministic for identical
 * inputs and arguments.
 *
 * Execution: one forward kernel on `stream` (preceded by a fill kernel only when the
 * library allocates the workspace itself) in which each workgroup loads R consecutive
 * chunks of one head (a "sweep") into shared memory, publishes that sweep's Fenwick
 * node in the workspace and reads the nodes of earlier sweeps of its head, waiting for
 * them with bounded polls. Workgroups are ordered by an atomic ticket, so a workgroup
 * only ever waits for workgroups that started before it. Should a wait nevertheless
 * run out (a fault elsewhere, or a workspace that was not zero-filled), the affected
 * outputs are written as NaN and the kernel still completes.
 *
 * Errors: every function validates its arguments on the host before it touches the
 * device and returns a status code (LLA_OK or a negative LLA_ERR_*); nothing is
 * printed, nothing aborts, no exception crosses the ABI. Launches are asynchronous
 * on `stream`; faults during kernel execution surface at the caller's next
 * synchronisation of that stream. Functions are thread safe; the library keeps no
 * state between calls (per-call state lives in the workspace).
 */
#ifndef LOGLINEAR_ATTN_H
#define LOGLINEAR_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t without pulling in the HIP headers. */
typedef struct ihipStream_t* lla_stream_t;

enum lla_status {
  LLA_OK = 0,
  LLA_ERR_INVALID_ARG = -1,   /* null pointer, negative size, aliasing out, bad struct */
  LLA_ERR_UNSUPPORTED = -2,   /* dk/dv/chunk/sweep outside the supported set, L > 24, B*H > 65535 */
  LLA_ERR_HIP = -3,           /* a HIP runtime call or a kernel launch failed */
  LLA_ERR_NO_MEMORY = -4,     /* stream-ordered workspace allocation failed (also forced, for
                                 tests, by LLA_TEST_FAIL_ALLOC=1 in the environment) */
  LLA_ERR_WORKSPACE = -5,     /* caller workspace smaller than loglinear_attn_workspace_bytes */
  LLA_ERR_SCRATCH_LIMIT = -6  /* loglinear_attn_fwd_noalloc: the call needs more workspace than
                                 its fixed scratch (loglinear_attn_noalloc_scratch_bytes) */
};

enum lla_dtype {
  LLA_DTYPE_BF16 = 0,         /* q, k, v, out bfloat16 */
  LLA_DTYPE_F32 = 1           /* q, k, v, out float32 */
};

/*
 * loglinear_attn_fwd — the forward pass with bfloat16 q, k, v, out.
 * log_a [B,H,T] and lambda [B,H,T,L] are float32. Chunk size and the number of
 * chunks one workgroup sweeps are chosen by the library. A workspace is taken
 * stream-ordered on `stream` (hipMallocAsync / hipFreeAsync) when the sequence
 * spans more than one sweep.
 * Returns LLA_OK or a negative LLA_ERR_* (see enum lla_status).
 */
int loglinear_attn_fwd(const void* q, const void* k, const void* v,
                       const float* log_a, const float* lambda, void* out,
                       int B, int H, int T, int dk, int dv, lla_stream_t stream);

/* loglinear_attn_fwd_f32 — the same operation with float32 q, k, v, out. */
int loglinear_attn_fwd_f32(const float* q, const float* k, const float* v,
                           const float* log_a, const float* lambda, float* out,
                           int B, int H, int T, int dk, int dv, lla_stream_t stream);

/*
 * Extended entry: explicit dtype, chunk size, sweep length and workspace.
 *   chunk : 0 = library default, else one of 16, 32, 64, 128.
 *   sweep : 0 = library default, else the number of consecutive chunks one
 *           workgroup holds in shared memory at once (1 or 2; LLA_ERR_UNSUPPORTED
 *           when they do not fit the device's shared memory).
 *   workspace / workspace_bytes : caller-owned device memory of at least
 *           loglinear_attn_workspace_bytes(...) bytes (256-byte aligned), or
 *           NULL/0 to let the library allocate (and zero) it stream-ordered on
 *           `stream`. A caller workspace must be zero-filled once before its first
 *           use (e.g. allocated zeroed); every call leaves it ready for the next one,
 *           whatever the shapes, so it is never cleared again. It holds the ticket
 *           counter (an epoch and a count), node flags and nodes of the running call:
 *           two calls that may run concurrently (different streams) must not share
 *           it; calls ordered on one stream may. Layout: the first
 *           round_up_256(4 * (64 + B*H*(nsweep-1)*dv/16)) bytes are the counter and
 *           flags, the only part that must start at zero. A workspace that was never
 *           zero-filled gives undefined outputs, but never leaves `out` unwritten: where
 *           the counter's count is at or past the number of workgroups every output row is
 *           written as NaN (and stays so on every later call until the workspace is
 *           zero-filled); where a node never comes, the rows that need it are NaN after a
 *           bounded wait.
 *   stage_events : optional timing hooks; each non-NULL entry is a hipEvent_t the
 *           library records on `stream`: [0] before the fill kernel (if any), [1]
 *           just before the forward kernel, [2] after it; [3] is not used. The caller
 *           owns the events.
 *   lambda_bf16 : 0 = lambda is float32 (4-byte aligned); 1 = lambda is bfloat16 (2-byte
 *           aligned, same [B,H,T,L] layout), read exactly and widened to float32 inside the
 *           kernel: the level weights then cost 2L instead of 4L bytes per head-token (the
 *           study notes list the lambda parameterisation among the things to check, section
 *           4-5). Any other value is LLA_ERR_INVALID_ARG.
 * The result does not depend on chunk or sweep beyond float rounding.
 */
typedef struct lla_fwd_args {
  const void* q;
  const void* k;
  const void* v;
  const float* log_a;
  const void* lambda;         /* float32, or bfloat16 when lambda_bf16 = 1 */
  void* out;
  int B, H, T, dk, dv;
  int dtype;                  /* enum lla_dtype */
  int chunk;
  int sweep;
  void* workspace;
  size_t workspace_bytes;
  void* stage_events[4];      /* hipEvent_t or NULL */
  int lambda_bf16;            /* 0: float32 lambda; 1: bfloat16 lambda */
} lla_fwd_args;

int loglinear_attn_fwd_ex(const lla_fwd_args* args, lla_stream_t stream);

/*
 * loglinear_attn_fwd_noalloc — loglinear_attn_fwd_ex that allocates nothing, for callers that
 * cannot allocate device memory around the call: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. The workspace lives in a fixed scratch array in the
 * library's device memory (loglinear_attn_noalloc_scratch_bytes() bytes, 64 MiB), one per
 * device, held from the first call on that device until the process ends; no hipMalloc,
 * hipFree or allocating library routine is called.
 *   args : as for loglinear_attn_fwd_ex, except that workspace must be NULL and workspace_bytes
 *          0 (LLA_ERR_INVALID_ARG otherwise). stage_events [1] and [2] are recorded around the
 *          forward kernel as there; [0] is recorded first.
 * Returns LLA_ERR_SCRATCH_LIMIT when loglinear_attn_workspace_bytes(...) for these arguments
 * exceeds the scratch (checked on the host before any device call); otherwise as
 * loglinear_attn_fwd_ex, with bitwise the same output.
 * The first call on a device also zero-fills the scratch with a fill kernel on `stream`. Every
 * call on a device shares that device's scratch and leaves it ready for the next call: calls on
 * one device that may overlap in time (different streams, threads or processes sharing a
 * context) race on it and must be serialised by the caller, e.g. by issuing them on one stream.
 */
int loglinear_attn_fwd_noalloc(const lla_fwd_args* args, lla_stream_t stream);

/* Size in bytes of the fixed scratch of loglinear_attn_fwd_noalloc (per device). */
size_t loglinear_attn_noalloc_scratch_bytes(void);

/*
 * loglinear_attn_fwd_varlen — the forward pass over a variable-length batch: N independent
 * sequences packed along the time axis. Sequence n of head h is rows
 * [cu_seqlens[n], cu_seqlens[n+1]) of the packed tensors; its positions restart at 0, so its
 * levels and decays are those of a batch of one sequence of length T_n (the operation above,
 * per sequence). Layout: dense row-major [H, total_T, .]:
 *   q, k [H, total_T, dk]   v, out [H, total_T, dv]   log_a [H, total_T]
 *   lambda [H, total_T, L], L = loglinear_attn_num_levels(max_T) (a sequence reads levels
 *   0 .. num_levels(T_n)-1 of its rows)
 *   cu_seqlens: device int32 [N+1], cu_seqlens[0] = 0, nondecreasing, cu_seqlens[N] =
 *   total_T, and no sequence longer than max_T (host value, sizes the workspace). The device
 *   array is not checked; the kernel clamps each sequence into the packed rows and to max_T,
 *   so a malformed array gives wrong outputs, never an access out of bounds. Rows outside
 *   every sequence are left as they were.
 *   cu_seqlens_host: NULL, or a host copy of the same N+1 values, read before the call
 *   returns; the launch then has exactly one workgroup per (sweep, sequence, head) that
 *   exists. Without it the grid is sized for N x H heads of max_T tokens and the surplus
 *   workgroups leave at once, which costs time when lengths vary a lot. The two copies must
 *   hold the same values: where they do not, the kernel sees it and writes no output.
 * Chunk, sweep, workspace: as in loglinear_attn_fwd_ex, with the shapes of N x H heads of
 * max_T tokens: the workspace needed is loglinear_attn_workspace_bytes(N, H, max_T, dk, dv,
 * chunk, sweep, dtype).
 */
typedef struct lla_fwd_varlen_args {
  const void* q;
  const void* k;
  const void* v;
  const float* log_a;
  const void* lambda;         /* float32, or bfloat16 when lambda_bf16 = 1 */
  void* out;
  const int* cu_seqlens;      /* device */
  const int* cu_seqlens_host; /* host copy, or NULL */
  int N, H, total_T, max_T, dk, dv;
  int dtype;                  /* enum lla_dtype */
  int chunk;
  int sweep;
  void* workspace;
  size_t workspace_bytes;
  int lambda_bf16;            /* as in lla_fwd_args */
} lla_fwd_varlen_args;

int loglinear_attn_fwd_varlen(const lla_fwd_varlen_args* args, lla_stream_t stream);

/*
 * Bytes of workspace loglinear_attn_fwd_ex needs for these arguments (0 when
 * the sequence fits one sweep). chunk/sweep 0 mean the library defaults, as in
 * loglinear_attn_fwd_ex. Returns 0 as well for invalid arguments; the entry
 * point reports those.
 */
size_t loglinear_attn_workspace_bytes(int B, int H, int T, int dk, int dv,
                                      int chunk, int sweep, int dtype);

/* Number of lambda levels for T tokens: bit_length(T-1) + 1 (1 for T = 1, 0 for T <= 0). */
int loglinear_attn_num_levels(int T);

/*
 * Chunk size and sweep length the library picks when both are left at 0 (0 for invalid
 * arguments), a rule fitted to forward-kernel times measured on MI355X over every chunk and sweep
 * that fits, at 17 shapes:
 *   chunk: 64; 128 for bfloat16 with dk = dv = 128 and T >= 65536; 32 for float32 with
 *          dk, dv <= 16;
 *   sweep: 2 for bfloat16 when the sequence has more than one chunk, two chunks fit the shared
 *          memory and B*H*ceil(chunks/2) >= 128 workgroups result; 1 otherwise (always 1 for
 *          float32).
 */
int loglinear_attn_default_chunk(int dk, int dv, int T, int dtype);
int loglinear_attn_default_sweep(int B, int H, int T, int dk, int dv, int chunk, int dtype);

/* Static, NUL-terminated description of a status code. */
const char* loglinear_attn_status_string(int status);

/*
 * loglinear_attn_decode_step — one decoding step: the same operator, one new token at position
 * t for every (b, h), through the recurrent form with one dk x dv state per Fenwick level
 * (study notes, sections 2-2 and 3-6; zh lay summary, "drawer" merging). With c = ctz(t) for
 * t > 0, the level states 0..c after position t-1 merge into level c+1, every state is
 * multiplied by a_t = exp(log_a_t), level 0 becomes k_t v_t^T, and
 *     o_t = sum_l lambda[l] * S_l^T q_t  over the levels live after t
 * (level 0 and level j+1 for each set bit j of t). Calling it for t = 0, 1, ..., T-1 on one
 * cache gives the forward pass's outputs for those positions.
 *
 *   q, k   [B,H,dk]  v, out [B,H,dv]   bfloat16 (dtype LLA_DTYPE_BF16) or float32
 *   log_a  [B,H]     lambda [B,H,Lc]  float32; lambda[.., l] = the token's weight of level l
 *                                      (levels above bit_length(t) are not read)
 *   state  [B,H,Lc,dk,dv] float32, log_scale [B,H,2,Lc] float32: the cache, owned by the
 *          caller and updated in place. Level l >= 1, while live, is
 *          state[b,h,l] * exp(log_scale[b,h,t&1,l]); level 0 (rank one) is kept as its
 *          factors: (k, v) of the last even position in floats [0, dk+dv) of state[b,h,0],
 *          of the last odd position in [dk+dv, 2(dk+dv)). Nothing is read before it was
 *          written, so the cache needs no clearing before t = 0.
 *   Lc     levels of the cache: at least bit_length(t) + 1 (LLA_ERR_INVALID_ARG otherwise),
 *          at most 25 (positions below 2^24).
 * Steps on one cache must run in order of t (on one stream).
 *   t_seq  NULL: every (b, h) is at position t. Else a device array of B int64 positions, one per
 *          sequence (a batch of prompts of different lengths decoded together; the heads of a
 *          sequence share its position), and t is the largest of them (it sizes the Lc check).
 *          A negative entry means that sequence takes no step: its cache and its out rows are
 *          left untouched (e.g. a finished request). An entry past t makes that sequence's out
 *          rows NaN and leaves its cache untouched, so a wrong array never reaches past the
 *          cache. 8-byte aligned; read on the device, never on the host.
 * Pointers are device pointers; out, state and log_scale must not overlap each other or the
 * inputs. Returns LLA_OK or a negative LLA_ERR_* (B*H = 0 is a no-op).
 */
typedef struct lla_decode_args {
  const void* q;
  const void* k;
  const void* v;
  const float* log_a;
  const float* lambda;
  void* out;
  float* state;
  float* log_scale;
  int B, H, dk, dv, Lc;
  int dtype;                  /* enum lla_dtype */
  long long t;
  const long long* t_seq;     /* per-sequence positions [B] (device), or NULL */
} lla_decode_args;

int loglinear_attn_decode_step(const lla_decode_args* args, lla_stream_t stream);

/*
 * loglinear_attn_decode_prefill — hand-over from a prompt of T tokens to the decoding step: fills
 * the cache so that loglinear_attn_decode_step can be called for t = T, T+1, ... and gives the
 * outputs of the forward pass over the prompt followed by the decoded tokens. After position
 * P = T - 1 the live levels are 0 (position P) and l = j + 1 for each set bit j of P, holding the
 * aligned block of 2^j positions [(P >> l) << l, + 2^j), decayed to P (study notes, sections 2-2
 * and 3-6): S_l = sum_{s in block} exp(A_P - A_s) k_s v_s^T.
 *   k [B,H,T,dk], v [B,H,T,dv]: bfloat16 (LLA_DTYPE_BF16) or float32, 16-byte aligned;
 *   log_a [B,H,T] float32.
 *   state [B,H,Lc,dk,dv], log_scale [B,H,2,Lc]: the decoding cache (float32, owned by the caller,
 *   layout as in loglinear_attn_decode_step); written: the live levels of P (unscaled), the
 *   level-0 factors of parity P & 1 and the log-scale row of that parity; nothing else is read.
 *   Lc >= bit_length(T) + 1 (the levels the step at t = T needs), <= 25.
 * Blocks longer than 256 positions are contracted in segments of 256 whose partial states go
 * to a scratch array the library allocates stream-ordered on `stream` (B*H*dk*dv*4 bytes per
 * segment; LLA_ERR_NO_MEMORY if that fails) and are then added in segment order.
 * Returns LLA_OK or a negative LLA_ERR_*; B*H = 0 is a no-op. Asynchronous on `stream`,
 * deterministic.
 */
typedef struct lla_prefill_args {
  const void* k;
  const void* v;
  const float* log_a;
  float* state;
  float* log_scale;
  int B, H, T, dk, dv, Lc;
  int dtype;                  /* enum lla_dtype */
} lla_prefill_args;

int loglinear_attn_decode_prefill(const lla_prefill_args* args, lla_stream_t stream);

/*
 * loglinear_attn_bwd — the backward pass: gradients of sum(grad_out * o) with respect to every
 * input of the forward operation above (the study notes name training speed and the gradient of
 * the level weights as the hard part of the method, sections 3-5 and 4-5). Per head, with
 * M[t,s] = lambda[t, l(t,s)] * exp(A_t - A_s) for s <= t, S[t,s] = q_t . k_s and
 * W[t,s] = grad_out_t . v_s:
 *   grad_q_t = sum_s M W k_s      grad_k_s = sum_t M W q_t      grad_v_s = sum_t M S grad_out_t
 *   grad_lambda[t, l] = sum over the s with l(t,s) = l of exp(A_t - A_s) S W  (0 for a level no
 *                       pair of row t reaches)
 *   grad_log_a[r] = sum_{t >= r} (q_t . grad_q_t - k_t . grad_k_t)
 *
 *   q, k [B,H,T,dk]  v, grad_out [B,H,T,dv]  bfloat16 (LLA_DTYPE_BF16) or float32, all alike
 *   log_a [B,H,T], lambda [B,H,T,L] float32, L = loglinear_attn_num_levels(T)
 *   grad_q, grad_k [B,H,T,dk], grad_v [B,H,T,dv] in q's dtype; grad_log_a [B,H,T] and
 *   grad_lambda [B,H,T,L] float32. All outputs are fully overwritten, never accumulated into.
 *   chunk : 0 = library default (loglinear_attn_bwd_default_chunk), else 16, 32 or 64
 *           (LLA_ERR_UNSUPPORTED when the gradient kernel's shared memory would exceed 160 KB).
 *   workspace / workspace_bytes : caller device memory of at least
 *           loglinear_attn_bwd_workspace_bytes(...) bytes (256-byte aligned; no clearing needed:
 *           every byte read was written earlier in the same call), or NULL/0 to let the library
 *           take it stream-ordered on `stream`. It holds the chunk-level Fenwick nodes, their
 *           log decays, the per-level partial states of the target side and the per-position
 *           dA of the running call, so calls that may run concurrently must not share it.
 *   stage_events : optional hipEvent_t the library records on `stream`: [0] before the chunk
 *           states, [1] before the gradient kernel, [2] after it, [3] after the grad_log_a scan.
 *   lambda_bf16 : 0 = lambda float32; 1 = lambda bfloat16 (2-byte aligned), read exactly as in
 *           loglinear_attn_fwd_ex; grad_lambda is float32 either way.
 * Pointers are device pointers; q, k, v, grad_out 16-byte aligned, the float arrays 4-byte
 * aligned; no output may overlap an input or another output (LLA_ERR_INVALID_ARG). Supported
 * shapes as for the forward pass (dk, dv in {16,32,64,128}, T < 2^23, B*H <= 65535).
 * Asynchronous on `stream`, bitwise deterministic, returns LLA_OK or a negative LLA_ERR_*.
 */
typedef struct lla_bwd_args {
  const void* q;
  const void* k;
  const void* v;
  const float* log_a;
  const void* lambda;         /* float32, or bfloat16 when lambda_bf16 = 1 */
  const void* grad_out;
  void* grad_q;
  void* grad_k;
  void* grad_v;
  float* grad_log_a;
  float* grad_lambda;
  int B, H, T, dk, dv;
  int dtype;                  /* enum lla_dtype */
  int chunk;
  void* workspace;
  size_t workspace_bytes;
  void* stage_events[4];      /* hipEvent_t or NULL */
  int lambda_bf16;            /* 0: float32 lambda; 1: bfloat16 lambda (grad_lambda stays float32) */
} lla_bwd_args;

int loglinear_attn_bwd(const lla_bwd_args* args, lla_stream_t stream);

/* Bytes of workspace loglinear_attn_bwd needs (0 for invalid or unsupported arguments). */
size_t loglinear_attn_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk,
                                          int dtype);

/* Chunk size loglinear_attn_bwd uses when chunk is 0 (0 for unsupported arguments). */
int loglinear_attn_bwd_default_chunk(int dk, int dv, int dtype);

/*
 * loglinear_attn_gdn_fwd — the forward pass of log-linear Gated DeltaNet: the Fenwick
 * hierarchical mask applied to Gated DeltaNet's own attention matrix, so that every level state
 * is carried by the delta-rule transition (study notes, section 3-5, where the model's temporal
 * mask is composed with the hierarchical one keeping its transition; gist.science de technical
 * summary, where every variant is O = (A * M)V with per-level recurrent states and the delta rule
 * is combined with the hierarchical structure; zh technical summary, section 2.4). Per (b, h, t):
 *
 *   o_t = sum_{s <= t} lambda[t, l(t,s)] beta_s q_t^T A_t A_{t-1} ... A_{s+1} k_s v_s
 *   A_r = a_r (I - beta_r k_r k_r^T),  a_r = exp(log_a[r]),  l(t, s) = bit_length(t XOR s)
 *
 * With every lambda equal this is Gated DeltaNet, S_t = a_t (I - beta_t k_t k_t^T) S_{t-1} +
 * beta_t k_t v_t^T, o_t = S_t^T q_t. The delta rule's transition is a contraction only for
 * ||k|| <= 1 and beta in [0, 2]: callers L2-normalise the keys (not checked).
 *
 *   q, k [B,H,T,dk], v, out [B,H,T,dv]: bfloat16 or float32 (dtype), 16-byte aligned
 *   log_a, beta [B,H,T] float32; lambda [B,H,T,L] float32 (or bfloat16, lambda_bf16 = 1)
 *   chunk : 0 = loglinear_attn_gdn_default_chunk(dk, dv, dtype), else 16, 32 or 64 when the
 *           kernels' shared memory fits 160 KB (chunk 64 needs dk, dv <= 64).
 *   workspace / workspace_bytes : caller device memory of at least
 *           loglinear_attn_gdn_workspace_bytes(...) bytes (256-byte aligned, no clearing: every
 *           byte read is written earlier in the call), or NULL/0 to let the library take it
 *           stream-ordered on `stream`. Holds, in float32, the intra-chunk outputs, the query
 *           rows carried to their chunk's start and the Fenwick tree over chunks (each node's
 *           dk x dv state and dk x dk transition; for bfloat16 inputs with 32 <= dk <= 64 each
 *           node matrix as its high bf16 parts followed by its low parts, the same 4 bytes per
 *           element); calls that may run concurrently must not share it.
 *   stage_events : optional hipEvent_t recorded on `stream`: [0] before the per-chunk kernel,
 *           [1] before the tree up-sweep, [2] before the query kernel, [3] after it.
 * Products run on the matrix cores in float32, except for bfloat16 inputs with dk >= 32: there
 * the query and up-sweep kernels' run in split bf16 (high and low parts, three bf16 products
 * each), and, at chunk 32 or 64 where q and k fit as bf16 images, the per-chunk kernel's leaf
 * state and transition and its attention matrix times v take the high and low parts of one
 * operand against the other, exact in bf16 (two bf16 products each); the
 * launches are gdn_chunk (one workgroup per chunk and head), the up-sweep (two tree levels per
 * launch for dk <= 64, else one), and gdn_query. Asynchronous on `stream`,
 * deterministic; returns LLA_OK or a negative LLA_ERR_*; B*H*T = 0 is a no-op.
 */
typedef struct lla_gdn_args {
  const void* q;
  const void* k;
  const void* v;
  const float* log_a;
  const float* beta;
  const void* lambda;         /* float32, or bfloat16 when lambda_bf16 = 1 */
  void* out;
  int B, H, T, dk, dv;
  int dtype;                  /* enum lla_dtype */
  int chunk;
  void* workspace;
  size_t workspace_bytes;
  void* stage_events[4];      /* hipEvent_t or NULL */
  int lambda_bf16;
} lla_gdn_args;

int loglinear_attn_gdn_fwd(const lla_gdn_args* args, lla_stream_t stream);

/* Bytes of workspace loglinear_attn_gdn_fwd needs (0 for invalid or unsupported arguments). */
size_t loglinear_attn_gdn_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int dtype);

/* Chunk loglinear_attn_gdn_fwd uses when chunk is 0: 32 where it fits (every supported head
 * size; measured fastest or tied with the best at every measured shape), else 16. */
int loglinear_attn_gdn_default_chunk(int dk, int dv, int dtype);

#ifdef __cplusplus
}
#endif

#endif /* LOGLINEAR_ATTN_H */
