/*
 * ccv.h -- C ABI of libccv: the causal depthwise conv1d forward on AMD gfx950.
 *
 * The operation (Ch.5 "Dao forward CUDA implementation", section "How adjacent
 * threads and chunks exchange history", stencil equation for z_i, with the
 * argument meanings of Ch.4 "Dao interface and source map", section "Contract
 * of the full-sequence interface", argument table):
 *
 *   out[b,c,t] = act( bias[c] + sum_{k=0}^{K-1} keep(b,t,k) * w[c,k] * X~[b,c,t-K+1+k] )
 *
 *   - K in {2,3,4}; w[c,k] is ordered oldest -> current, so w[c,K-1] meets x[b,c,t].
 *   - X~[b,c,j] = x[b,c,j] for j >= 0.  For j < 0 it is the history left of the
 *     block: initial_states[b,c,j+K-1] (time ascending: index K-2 is t = -1) when
 *     given, otherwise 0 (Ch.5, section "Three kinds of boundary handled
 *     separately").
 *   - keep = 1 without seq_idx.  With seq_idx, a term counts only when its source
 *     step s = t-K+1+k is >= 0 and seq_idx[b,s] == seq_idx[b,t]; other terms are
 *     dropped (skipped, so a NaN in another sequence never reaches this one)
 *     (same section, seq_idx paragraph).  Ids are compared for equality only.
 *   - act is the identity or SiLU z*sigmoid(z) ("silu" and "swish" are the same
 *     activation), applied to the fp32 accumulator before the single rounding to
 *     the output dtype (Ch.5, same section as the stencil; Ch.4, section "How
 *     autograd links forward and backward", on result dtype vs accumulation dtype).
 *   - final_states_out[b,c,i] = X~[b,c,L-K+1+i], i = 0..K-2: the last K-1 conv
 *     inputs (not activations), copied bit for bit; correct for L < K-1 and L = 0
 *     (Ch.5, section "Three kinds of boundary handled separately").
 *   - seq_idx together with states (a limit of the pages' library version, not
 *     of the mathematics: Ch.4, section "Concrete limits of v1.5.0", lifted here):
 *     initial_states is the history of the row's first sequence, so a term
 *     reaching left of t = 0 counts when seq_idx[b,t] == seq_idx[b,0]; and
 *     final_states is the history of the row's last sequence, so an entry from
 *     another sequence is 0.  A packed row split anywhere then runs as two calls:
 *     pass the first call's final_states as the second's initial_states where
 *     the sequence continues across the split, zeros where one starts there.
 *
 * Layout: every tensor argument is a pointer plus element strides; the element
 * at (b,c,t) is at base + b*s_B + c*s_C + t*s_L elements (Ch.4, section "Why one
 * shape still has two layouts", offset equation).  x must have unit stride in
 * time (channel-first kernel) or in channels (channel-last kernel); a slice of a
 * wider projection buffer (s_L > C) is used as is, never repacked.  `out` must
 * have unit stride in the same dimension as x.
 *
 * Ownership: the caller allocates and owns every buffer (device memory for all
 * tensor pointers).  The library allocates nothing, keeps no pointer after a
 * call returns, never synchronises, and is safe to call concurrently on
 * different streams.  `out` must not overlap any input; views interleaved in one
 * parent buffer are fine as long as the elements touched are disjoint.
 *
 * Errors: every call returns a ccv_status (0 = success, negative = error).  All
 * argument checks run before anything is enqueued, so a call that fails writes
 * nothing.  No C++ exception crosses this boundary.
 */
#ifndef CCV_H
#define CCV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CCV_ABI_VERSION 1

/* Storage dtypes of x / out / states (x_dtype) and of weight / bias (w_dtype).
 * Ch.4, section "Concrete limits of v1.5.0": x and weight each take one of
 * fp32, fp16, bf16, dispatched separately; bias has the weight's dtype; states
 * have x's dtype. */
typedef enum { CCV_F32 = 0, CCV_F16 = 1, CCV_BF16 = 2 } ccv_dtype_t;

/* Activation flag (Ch.4, section "Contract of the full-sequence interface":
 * activation is none, "silu" or "swish"; the last two are one activation). */
typedef enum { CCV_ACT_NONE = 0, CCV_ACT_SILU = 1 } ccv_act_t;

typedef enum {
  CCV_OK = 0,
  CCV_E_NULL = -1,        /* a pointer the call needs is NULL */
  CCV_E_SHAPE = -2,       /* B, C or L negative, or sizes overflow int64 offsets */
  CCV_E_KSIZE = -3,       /* K not in {2,3,4} */
  CCV_E_DTYPE = -4,       /* x_dtype or w_dtype not a ccv_dtype_t */
  CCV_E_LAYOUT = -5,      /* x (or out) has unit stride in neither time nor channels,
                             out's unit-stride dim differs from x's, a stride < 0, or the
                             layout of out or final_states_out maps two elements to one
                             address */
  CCV_E_UNSUPPORTED = -6, /* an activation value outside ccv_act_t; in the backward,
                             dinitial_states without initial_states */
  CCV_E_ALIAS = -7,       /* out == x, or final_states_out is x, out or initial_states */
  CCV_E_HIP = -8,         /* the HIP runtime refused the launch */
  CCV_E_INTERNAL = -9,    /* an unexpected internal condition */
  CCV_E_ABI = -10,        /* struct_size does not match this library's struct */
  CCV_E_SCRATCH = -11     /* ccv_bwd_static: the call needs more partial-sum space than
                             the library's fixed array (CCV_BWD_STATIC_SCRATCH_BYTES) */
} ccv_status_t;

/* All arguments of one forward call.  Strides are in elements. */
typedef struct ccv_fwd_args {
  int64_t struct_size;          /* = sizeof(ccv_fwd_args_t) */
  int64_t B, C, L;              /* logical shape of x and out: [B, C, L] */
  int32_t K;                    /* taps: 2, 3 or 4 */
  int32_t activation;           /* ccv_act_t */
  int32_t x_dtype;              /* ccv_dtype_t of x, out, initial_states, final_states_out */
  int32_t w_dtype;              /* ccv_dtype_t of weight and bias */
  const void* x;                /* device, x[b,c,t] */
  int64_t x_stride[3];          /*   (s_B, s_C, s_L) */
  const void* weight;           /* device, contiguous [C, K], oldest -> current */
  const void* bias;             /* device [C] or NULL (pre-activation) */
  const int32_t* seq_idx;       /* device, contiguous int32 [B, L], or NULL */
  const void* initial_states;   /* device [B, C, K-1] or NULL (history left of t = 0) */
  int64_t init_stride[3];       /*   (b, c, i) strides */
  void* final_states_out;       /* device [B, C, K-1] or NULL (the last K-1 inputs) */
  int64_t final_stride[3];      /*   (b, c, i) strides */
  void* out;                    /* device [B, C, L] */
  int64_t out_stride[3];        /*   (s_B, s_C, s_L) */
} ccv_fwd_args_t;

/* Which kernel a call would launch and how (host-only; for tests and benches). */
typedef enum {
  CCV_PATH_NONE = 0, CCV_PATH_CHANNEL_FIRST = 1, CCV_PATH_CHANNEL_LAST = 2,
  CCV_PATH_UPDATE = 3,     /* the update (decode) kernel; see ccv_update_plan */
  CCV_PATH_BACKWARD = 4    /* the backward kernels; see ccv_bwd_plan */
} ccv_path_t;

typedef struct ccv_plan {
  int32_t path;            /* ccv_path_t; NONE when there is nothing to compute or write */
  int32_t vector;          /* 1: 16-byte loads and stores; 0: element loads and stores.
                              Channel-first rows take 16-byte accesses at any length and
                              element offset (the vector that straddles L moves element by
                              element); channel-last whole channel vectors too (a
                              lane's partial vector moves element by element) */
  int32_t elems_per_lane;  /* elements one lane holds per 16-byte vector (16 / element size) */
  int32_t unroll;          /* vectors (channel-first) or time rows (channel-last) in flight per
                              lane; channel-last: 8 when whole tiles take the straight-line
                              path (the row batch being computed and the next one; weights,
                              bias, history rows and seq_idx ids as vectors), 4 otherwise */
  int64_t grid;            /* workgroups launched (channel-first with L not a multiple of
                              span: the whole segments' workgroups, then one wave per row for
                              the row's last, shorter segment) */
  int32_t block;           /* threads per workgroup */
  int32_t waves_per_group; /* independent wave work items per workgroup */
  int64_t work_items;      /* wave work items (channel-first: B*C rows times ceil(L / span)
                              segments; otherwise grid * waves_per_group rounded down to the
                              need) */
  int64_t span;            /* channel-first: time steps per work item; channel-last: time rows per work item */
  int64_t channels_per_item; /* channel-last: channels per work item; channel-first: 1 */
} ccv_plan_t;

/* Enqueue the forward on `hip_stream` (a hipStream_t; NULL = the null stream) and
 * return without waiting.  Returns CCV_OK, a validation error (nothing enqueued)
 * or CCV_E_HIP (also when the runtime cannot name the stream's GPU).  Faults of
 * the kernel itself surface at the caller's next synchronisation of that stream.
 * The grid is sized for the stream's GPU: its compute-unit count is read from the
 * runtime on the first call on that GPU and kept; the environment variable
 * CCV_CU_COUNT, when set to a positive count, replaces it. */
int ccv_fwd(const ccv_fwd_args_t* args, void* hip_stream);

/* Launch tuning and ablation switches, read from the environment at each call of
 * ccv_fwd / ccv_fwd_plan (none is needed; every setting gives the same results,
 * bit for bit):
 *   CCV_CU_COUNT=n         size grids for n compute units (see ccv_fwd).
 *   CCV_CF_WAVES_PER_CU=n  channel-first: a grid of n waves per compute unit, each
 *                          walking several segments (0: one wave per segment).
 *   CCV_CL_WAVES_PER_CU=n  channel-last: the same for tiles (default 0).
 *   CCV_CL_TILE_T=n        channel-last: time rows per tile (default 32, at least 4).
 *   CCV_CL_LDS=1 | 2       channel-last: tiles staged through LDS (16 rows), or the
 *                          transposing tile of 256 channels (16-byte aligned
 *                          rows only, and C a multiple of 16 / element size for
 *                          the transposing tile; others keep the default path).
 *   CCV_FORCE_SCALAR=1     element-wise loads and stores (read by ccv_update and
 *                          ccv_bwd too; the backward's dweight and dbias are then
 *                          summed in another fixed order, so they agree to rounding).
 * The plan (ccv_fwd_plan) shows the launch they lead to. */

/* Validate `args` exactly as ccv_fwd does, without touching any device. */
int ccv_fwd_check(const ccv_fwd_args_t* args);

/* Validate and describe the launch ccv_fwd would make, without touching any
 * device: the grid is sized for the GPU of the latest ccv_fwd call in this process
 * (for 256 compute units, MI355X's count, before any; CCV_CU_COUNT as above).
 * `plan` may be NULL. */
int ccv_fwd_plan(const ccv_fwd_args_t* args, ccv_plan_t* plan);

/* ---- update (decode): advance a K-1 step history in place ------------------------
 *
 * The step after a forward over a prompt: a few new steps per (b, c) row are
 * convolved against the history that precedes them, and the history is then
 * replaced by the last K-1 inputs, in the same buffer (Ch.4 "Dao interface and
 * source map", section "Reading the source along the call chain": the update
 * kernel reads the history and advances the state in place).  With
 * X~ = state[b,c,0..K-2] followed by x[b,c,0..L-1]:
 *
 *   out[b,c,t]   = act( bias[c] + sum_{k=0}^{K-1} w[c,k] * X~[t+k] ),  t = 0..L-1
 *   state[b,c,i] <- X~[L+i],                                           i = 0..K-2
 *
 * which is exactly ccv_fwd with initial_states = final_states_out = state (the
 * stencil of Ch.5 "Dao forward CUDA implementation", section "How adjacent
 * threads and chunks exchange history"; the state as the history left of the
 * block and as the last K-1 inputs, Ch.5, section "Three kinds of boundary
 * handled separately").  The arithmetic is the forward's, term for term and in
 * the same order, so decoding one step at a time gives the forward's bits.
 * There is no seq_idx: every row is one sequence.  Any L works, but each row is
 * processed sequentially by one thread, so long runs belong to ccv_fwd.
 *
 * state is read before it is written, row by row, so it is updated in place;
 * it must not overlap x or out, and the state and out layouts must not map two
 * logical elements to one address (CCV_E_LAYOUT).  L = 0 leaves state as it is
 * and enqueues nothing.  Any element strides are accepted for every tensor. */
typedef struct ccv_update_args {
  int64_t struct_size;          /* = sizeof(ccv_update_args_t) */
  int64_t B, C, L;              /* x and out: [B, C, L] new steps (decode: L = 1) */
  int32_t K;                    /* taps: 2, 3 or 4 */
  int32_t activation;           /* ccv_act_t */
  int32_t x_dtype;              /* ccv_dtype_t of x, out and state */
  int32_t w_dtype;              /* ccv_dtype_t of weight and bias */
  const void* x;                /* device, x[b,c,t] */
  int64_t x_stride[3];          /*   (s_B, s_C, s_L) */
  const void* weight;           /* device, contiguous [C, K], oldest -> current */
  const void* bias;             /* device [C] or NULL (pre-activation) */
  void* state;                  /* device [B, C, K-1], time ascending; read, then overwritten */
  int64_t state_stride[3];      /*   (b, c, i) strides */
  void* out;                    /* device [B, C, L] */
  int64_t out_stride[3];        /*   (s_B, s_C, s_L) */
} ccv_update_args_t;

/* Enqueue one update on `hip_stream` (NULL = the null stream) and return without
 * waiting.  Returns CCV_OK, a validation error (nothing enqueued) or CCV_E_HIP.
 * Errors: CCV_E_NULL (x, weight, state or out missing when B*C*L > 0),
 * CCV_E_SHAPE, CCV_E_KSIZE, CCV_E_DTYPE, CCV_E_UNSUPPORTED (activation value),
 * CCV_E_ALIAS (any two of x, state, out share a base address), CCV_E_LAYOUT (a
 * negative stride, or a state / out layout that overlaps itself), CCV_E_ABI. */
int ccv_update(const ccv_update_args_t* args, void* hip_stream);

/* Validate `args` exactly as ccv_update does, without touching any device. */
int ccv_update_check(const ccv_update_args_t* args);

/* Validate and describe the launch ccv_update would make, without touching any
 * device (`plan` may be NULL): path CCV_PATH_UPDATE (NONE when nothing is
 * enqueued); vector 1 when each lane moves whole 16-byte vectors of V = 16 /
 * element size consecutive channels (C a multiple of V, x and out unit-stride in
 * channels, the state stored [B, C, K-1] contiguously, all 16-byte aligned;
 * weight and bias of any dtype), else 0; elems_per_lane and
 * channels_per_item: rows per lane; grid, block, waves_per_group: the launch;
 * work_items: B*C rows; span: L; unroll: 1. */
int ccv_update_plan(const ccv_update_args_t* args, ccv_plan_t* plan);

/* ---- backward -----------------------------------------------------------------------
 *
 * The gradients of ccv_fwd (Ch.4 "Dao interface and source map", section "How
 * autograd links forward and backward": the backward receives dout and, when the
 * forward returned final states, dfinal_states; it returns dx, dweight, dbias and
 * the gradient of initial_states; dweight and dbias are accumulated in fp32 and
 * converted to the parameter dtype at the end; seq_idx has no gradient).  With z
 * the pre-activation (recomputed, not stored) and X~ the extended input:
 *
 *   dz[b,c,t]   = dout[b,c,t] * act'(z[b,c,t])          (SiLU': s(z) (1 + z (1 - s(z))))
 *   dX~[b,c,j]  = sum_k keep(t,k) w[c,k] dz[b,c,t] over t = j+K-1-k in [0, L)
 *                 + dfinal_states[b,c,j-(L-K+1)]  when j >= L-K+1
 *   dx[b,c,t]   = dX~[b,c,t];   dinitial_states[b,c,i] = dX~[b,c,i-(K-1)]
 *   dweight[c,k] = sum_{b,t} keep(t,k) dz[b,c,t] X~[b,c,t-K+1+k];  dbias[c] = sum_{b,t} dz[b,c,t]
 *
 * Every sum is fp32; dx and dinitial_states are rounded once to x's dtype,
 * dweight and dbias once to the weight dtype.  The parameter sums run in a fixed
 * order (within each group of consecutive time tiles of a row, then over the groups
 * by a tree of fixed shape), so results repeat bit for bit.  With
 * seq_idx, keep() and the history's sequence are the forward's, and
 * dfinal_states reaches only the entries that final_states kept.  Any element strides are accepted for x,
 * dout, dx and the states; weight, bias, dweight, dbias are contiguous.  dx must
 * not be x or dout; dinitial_states must not be initial_states (CCV_E_ALIAS).
 *
 * Workspace: the fp32 partial sums of dweight and dbias live in a caller-provided
 * device buffer of ccv_bwd_workspace_size(args) bytes (16-byte aligned; its
 * contents on entry do not matter).  It is CCV_E_NULL to pass none when that size
 * is nonzero and CCV_E_SHAPE to pass fewer bytes. */
typedef struct ccv_bwd_args {
  int64_t struct_size;          /* = sizeof(ccv_bwd_args_t) */
  int64_t B, C, L;              /* logical shape of x, dout, dx: [B, C, L] */
  int32_t K;                    /* taps: 2, 3 or 4 */
  int32_t activation;           /* ccv_act_t of the forward */
  int32_t x_dtype;              /* of x, dout, dx, the states and their gradients */
  int32_t w_dtype;              /* of weight, bias, dweight, dbias */
  const void* x;                /* device, the forward's input */
  int64_t x_stride[3];
  const void* weight;           /* device, contiguous [C, K] */
  const void* bias;             /* device [C] or NULL: the forward's bias (needed to recompute z) */
  const int32_t* seq_idx;       /* device, contiguous int32 [B, L], or NULL */
  const void* initial_states;   /* device [B, C, K-1] or NULL: the forward's history */
  int64_t init_stride[3];
  const void* dout;             /* device [B, C, L]: gradient of out */
  int64_t dout_stride[3];
  const void* dfinal_states;    /* device [B, C, K-1] or NULL: gradient of final_states */
  int64_t dfinal_stride[3];
  void* dx;                     /* device [B, C, L] */
  int64_t dx_stride[3];
  void* dweight;                /* device, contiguous [C, K] */
  void* dbias;                  /* device [C] or NULL (not computed) */
  void* dinitial_states;        /* device [B, C, K-1] or NULL; needs initial_states */
  int64_t dinit_stride[3];
  void* workspace;              /* device scratch, ccv_bwd_workspace_size bytes */
  int64_t workspace_bytes;
} ccv_bwd_args_t;

/* Bytes of workspace ccv_bwd needs for `args` (>= 0), or a negative status when
 * the arguments are invalid.  Host only. */
int64_t ccv_bwd_workspace_size(const ccv_bwd_args_t* args);

/* Enqueue the backward (the gradient kernel, then one kernel per level of the
 * reduction tree, in order) on `hip_stream` and return without waiting.  Returns CCV_OK, a validation error (nothing enqueued) or CCV_E_HIP. */
int ccv_bwd(const ccv_bwd_args_t* args, void* hip_stream);

/* Validate `args` exactly as ccv_bwd does, without touching any device. */
int ccv_bwd_check(const ccv_bwd_args_t* args);

/* Describe the launch ccv_bwd would make (host only; `plan` may be NULL): path
 * CCV_PATH_BACKWARD; vector 0 for the element path (one lane per (b, tile group, c),
 * any strides), 1 for the LDS-staged channel-first path (used when seq_idx is not
 * 16-byte aligned), 2 for the LDS-staged channel-last path, 3 for the
 * register-only channel-first path (with or without seq_idx: one wave per (b, c,
 * segment of `span` steps), one partial row per (b, segment), elems_per_lane =
 * 16 / element size); the channel-first paths need x, dout and dx unit-stride in
 * time, the channel-last one in channels.  The register path and the channel-last
 * path take rows of any length and offset (unaligned 16-byte accesses, the vector
 * that straddles L resp. C element by element); the LDS-staged channel-first path
 * (seq_idx not 16-byte aligned) needs 16-byte aligned rows with L a multiple of
 * 16 / element size.  span = time
 * steps per tile (per segment on path 3); unroll = consecutive tiles per work
 * item (summed into one partial row: 4 when x is unit-stride in channels, else 1);
 * channels_per_item = channels per work item; work_items, grid, block of the
 * gradient kernel.  The workspace fields are not checked here, so a plan can
 * be had before the workspace is allocated. */
int ccv_bwd_plan(const ccv_bwd_args_t* args, ccv_plan_t* plan);

/* ---- backward without allocation --------------------------------------------------
 *
 * For callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  ccv_bwd_static is ccv_bwd
 * with the fp32 partial sums in a fixed device array of the library instead of the
 * caller's workspace; the caller still passes (and owns) every input and output,
 * and args->workspace / workspace_bytes are ignored.  Same kernels, same launches,
 * same results bit for bit.
 *
 * The array holds CCV_BWD_STATIC_SCRATCH_BYTES (64 MiB, enough for every call
 * whose ccv_bwd_workspace_size is at most that: e.g. bf16 [8, 4096, 8192] needs
 * 40 MiB); a call that needs more returns CCV_E_SCRATCH and enqueues nothing.
 * Each GPU the library runs on holds its own array from the first call there until
 * the process ends.  The call allocates nothing (no hipMalloc, no hipFree); its
 * first call on a device looks up that device's array address once.  The stream
 * (NULL = the null stream of the current device) must belong to the current device,
 * else CCV_E_UNSUPPORTED.  Every call on one GPU shares that GPU's array: calls
 * that overlap in time on one GPU (on different streams, or from several host
 * threads without ordering) race on it and give wrong parameter gradients; calls
 * ordered on one stream are fine.  Nothing in the array needs clearing between
 * calls (each call writes every partial sum it reads).  Other errors as ccv_bwd. */
#define CCV_BWD_STATIC_SCRATCH_BYTES ((int64_t)64 << 20)
int ccv_bwd_static(const ccv_bwd_args_t* args, void* hip_stream);

/* Static, NUL-terminated name of a status code ("CCV_OK", ...). */
const char* ccv_status_str(int status);

/* CCV_ABI_VERSION of the loaded library. */
int ccv_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CCV_H */
