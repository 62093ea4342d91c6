// ccv_api.cpp -- the C ABI of libccv: argument checks, kernel choice, launch.
//
// The checks follow the contract of Ch.4 "Dao interface and source map"
// (section "Contract of the full-sequence interface", argument table; section
// "Concrete limits of v1.5.0": K in {2,3,4}, three storage dtypes for x and
// weight dispatched separately, bias in the weight dtype, states in x's dtype).
// That version's other limits are lifted, since the page calls them limits of
// the version and not of the mathematics: states and seq_idx work with either
// layout and with each other (the history is the row's first sequence's, the
// final states the row's last sequence's), and neither layout needs
// multiple-of-8 alignment (both take unaligned 16-byte accesses; a partial vector
// at a row's or a channel group's end moves element by element).
//
// Nothing here touches a device except ccv_fwd's kernel launches.
#include <stdint.h>
#include <stdlib.h>

#include "ccv.h"
#include "ccv_checks.hpp"
#include "ccv_launch.hpp"

namespace {

using namespace ccv;
using namespace ccv::checks;

struct Plan {
  ccv_plan_t pub;
  bool silu, seq;
  CfArgs cf;
  ClArgs cl;
};

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  if (!v || !*v) return dflt;
  return atoi(v);
}

// Checks every argument and fills *plan (never NULL) with the launch to make.
int validate(const ccv_fwd_args_t* a, Plan* plan, int cus) {
  if (!a) return CCV_E_NULL;
  if (a->struct_size != (int64_t)sizeof(ccv_fwd_args_t)) return CCV_E_ABI;
  if (a->B < 0 || a->C < 0 || a->L < 0) return CCV_E_SHAPE;
  if (a->C > INT32_MAX || a->L > INT32_MAX) return CCV_E_SHAPE;
  if (a->K < 2 || a->K > 4) return CCV_E_KSIZE;
  if (a->x_dtype < 0 || a->x_dtype > 2 || a->w_dtype < 0 || a->w_dtype > 2) return CCV_E_DTYPE;
  if (a->activation != CCV_ACT_NONE && a->activation != CCV_ACT_SILU) return CCV_E_UNSUPPORTED;
  for (int d = 0; d < 3; ++d) {
    if (a->x_stride[d] < 0 || a->out_stride[d] < 0) return CCV_E_LAYOUT;
    if (a->initial_states && a->init_stride[d] < 0) return CCV_E_LAYOUT;
    if (a->final_states_out && a->final_stride[d] < 0) return CCV_E_LAYOUT;
  }

  const int64_t B = a->B, C = a->C, L = a->L;
  const int K = a->K;
  int64_t rows;
  if (__builtin_mul_overflow(B, C, &rows)) return CCV_E_SHAPE;
  const bool want_out = B > 0 && C > 0 && L > 0;
  const bool want_fin = B > 0 && C > 0 && a->final_states_out != nullptr;
  *plan = Plan{};
  plan->pub.path = CCV_PATH_NONE;
  if (!want_out && !want_fin) return CCV_OK;

  if (want_out && (!a->x || !a->weight || !a->out)) return CCV_E_NULL;
  if (want_out && a->out == a->x) return CCV_E_ALIAS;
  if (a->final_states_out && a->initial_states && a->final_states_out == a->initial_states) return CCV_E_ALIAS;
  if (want_fin && (a->final_states_out == a->x || (want_out && a->final_states_out == a->out)))
    return CCV_E_ALIAS;

  // Kernel choice by the unit-stride dimension of x (Ch.4, section "Why one shape
  // still has two layouts"); out must be unit-stride in the same dimension.  The
  // stride of a dimension of size <= 1 is never used, so it matches either way.
  const bool x_cf = a->x_stride[2] == 1 || L <= 1, x_cl = a->x_stride[1] == 1 || C <= 1;
  const bool o_cf = !want_out || a->out_stride[2] == 1 || L <= 1;
  const bool o_cl = !want_out || a->out_stride[1] == 1 || C <= 1;
  int path;
  if (a->x_stride[2] == 1 && L > 1 && o_cf) path = CCV_PATH_CHANNEL_FIRST;
  else if (x_cl && o_cl) path = CCV_PATH_CHANNEL_LAST;
  else if (x_cf && o_cf) path = CCV_PATH_CHANNEL_FIRST;
  else return CCV_E_LAYOUT;

  const int es = elt_size(a->x_dtype);
  const int64_t nx[3] = {B, C, L}, ns[3] = {B, C, K - 1};
  const int64_t xo = max_offset(nx, a->x_stride);
  if (!fits_bytes(xo, es)) return CCV_E_SHAPE;
  if (want_out && !fits_bytes(max_offset(nx, a->out_stride), es)) return CCV_E_SHAPE;
  if (a->initial_states && !fits_bytes(max_offset(ns, a->init_stride), es)) return CCV_E_SHAPE;
  if (a->final_states_out && !fits_bytes(max_offset(ns, a->final_stride), es)) return CCV_E_SHAPE;
  int64_t bl;
  if (a->seq_idx && __builtin_mul_overflow(B, L, &bl)) return CCV_E_SHAPE;
  // Waves write out and final_states_out concurrently, each element once: a
  // layout that maps two logical elements to one address would race.
  if (want_out && !non_overlapping(nx, a->out_stride)) return CCV_E_LAYOUT;
  if (want_fin && !non_overlapping(ns, a->final_stride)) return CCV_E_LAYOUT;

  const int V = 16 / es;
  Common m{};
  m.x = a->x;
  m.out = want_out ? a->out : nullptr;
  m.w = a->weight;
  m.bias = a->bias;
  m.seq = a->seq_idx;
  m.init = a->initial_states;
  m.fin = a->final_states_out;
  m.B = B; m.C = C; m.L = L;
  m.is_b = a->init_stride[0]; m.is_c = a->init_stride[1]; m.is_i = a->init_stride[2];
  m.fs_b = a->final_stride[0]; m.fs_c = a->final_stride[1]; m.fs_i = a->final_stride[2];
  m.w_dtype = a->w_dtype;

  const bool force_scalar = env_int("CCV_FORCE_SCALAR", 0) != 0;
  ccv_plan_t& P = plan->pub;
  P.path = path;
  P.elems_per_lane = V;
  P.block = 64 * kWavesPerGroup;
  P.waves_per_group = kWavesPerGroup;
  plan->silu = a->activation == CCV_ACT_SILU;
  plan->seq = a->seq_idx != nullptr;
  int64_t nwork;
  int64_t tail_groups = 0;

  if (path == CCV_PATH_CHANNEL_FIRST) {
    CfArgs& c = plan->cf;
    c.x_sb = a->x_stride[0]; c.x_sc = a->x_stride[1];
    c.o_sb = a->out_stride[0]; c.o_sc = a->out_stride[1];
    c.span = (int64_t)64 * V * kCfUnroll;
    c.nseg = L > 0 ? (L + c.span - 1) / c.span : 1;
    // Rows of any length and element offset take the 16-byte path: gfx950 serves
    // 16-byte accesses at any element alignment (measured on MI355X: a bf16 copy
    // offset by 2 bytes moves 5330 GB/s against 6040 aligned, back to back), and the
    // one vector per row that straddles L moves element by element.
    const bool vec = !force_scalar;
    c.nfull = vec ? L / c.span : 0;
    if (__builtin_mul_overflow(rows, c.nseg, &nwork)) return CCV_E_SHAPE;
    // A row's last, shorter segment (L not a multiple of the span) runs in one wave
    // of its own in workgroups appended to the grid; the waves counted here take
    // the whole segments.
    const bool tails = vec && L > 0 && L % c.span != 0;
    const int64_t nmain = tails ? rows * c.nfull : nwork;
    // Waves launched.  Arithmetic-heavy calls (16-bit storage packs twice the
    // outputs into each byte; SiLU adds two transcendentals per output) run a grid
    // of 16 waves per CU, each walking its segments with the next one's loads in
    // flight during the current one's arithmetic.  Light calls (fp32, no
    // activation) get one wave per segment, which keeps the most loads in flight.
    // Measured on MI355X: bf16 + SiLU 5260 GB/s pipelined vs 5015 one wave per
    // segment; fp32 K=3 without activation 5910 vs 5660.  CCV_CF_WAVES_PER_CU
    // overrides the choice.
    const bool heavy = es == 2 || a->activation == CCV_ACT_SILU;
    const int wpc = env_int("CCV_CF_WAVES_PER_CU", heavy ? 16 : 0);
    const int64_t cap = wpc > 0 ? (int64_t)cu_count(cus) * wpc : nmain;
    c.nwaves = nmain < cap ? nmain : cap;
    tail_groups = tails ? (rows + kWavesPerGroup - 1) / kWavesPerGroup : 0;
    P.vector = vec;
    P.unroll = kCfUnroll;
    P.span = c.span;
    P.channels_per_item = 1;
  } else {
    ClArgs& c = plan->cl;
    c.x_sb = a->x_stride[0]; c.x_sl = a->x_stride[2];
    c.o_sb = a->out_stride[0]; c.o_sl = a->out_stride[2];
    // 32-row tiles: measured best on MI355X for the strided bf16 view (5690 GB/s vs
    // 4855 at 64 rows) and the packed fp16 call (5027 vs 4998).
    int tile = env_int("CCV_CL_TILE_T", 32);
    if (tile < kClUnroll) tile = kClUnroll;
    // CCV_CL_LDS=1: whole tiles staged through LDS, kClLdsRows rows each; =2: the
    // transposing tile of kClTrChannels channels (both measured against the register
    // path; neither is the default).
    const bool vec_x = aligned16(a->x) && stride_ok16(B, a->x_stride[0], es) && stride_ok16(L, a->x_stride[2], es) &&
                       (!want_out || (aligned16(a->out) && stride_ok16(B, a->out_stride[0], es) &&
                                      stride_ok16(L, a->out_stride[2], es)));
    c.lds = env_int("CCV_CL_LDS", 0);
    if (c.lds == 1 && !(vec_x && !force_scalar)) c.lds = 0;   // global-to-LDS loads: aligned rows
    if (c.lds == 2 && !(vec_x && C % V == 0 && !force_scalar)) c.lds = 0;
    if (c.lds != 1 && c.lds != 2) c.lds = 0;
    if (c.lds == 1) tile = kClLdsRows;
    if (c.lds == 2) tile = cl_tr_rows(es);
    c.tile = tile;
    c.ntt = L > 0 ? (L + tile - 1) / tile : 1;
    c.ncg = c.lds == 2 ? (C + kClTrChannels - 1) / kClTrChannels : (C + 64 * V - 1) / (64 * V);
    int64_t bcg;
    if (__builtin_mul_overflow(B, c.ncg, &bcg) || __builtin_mul_overflow(bcg, c.ntt, &nwork)) return CCV_E_SHAPE;
    // Whole channel vectors take 16-byte accesses at any alignment (time rows that
    // are not 16-byte aligned: C not a multiple of V, or an offset channel view);
    // a lane's last, partial channel vector moves element by element.
    P.vector = !force_scalar;
    // Whole tiles take 16-byte loads for the history rows from initial_states, the
    // rows of 4 sequence ids and each lane's weight / bias block when those are
    // aligned (otherwise those tiles take the general tile code).
    const int64_t* is = a->init_stride;
    c.vec_init = a->initial_states && is[1] == 1 && aligned16(a->initial_states) &&
                 stride_ok16(B, is[0], es) && stride_ok16(K - 1, is[2], es);
    c.vec_seq = a->seq_idx && aligned16(a->seq_idx) && (B <= 1 || (L & 3) == 0);
    c.vec_par = aligned16(a->weight) && (!a->bias || aligned16(a->bias));
    const int wpc = env_int("CCV_CL_WAVES_PER_CU", 0);
    const int64_t cap = wpc > 0 ? (int64_t)cu_count(cus) * wpc : nwork;
    c.nwaves = nwork < cap ? nwork : cap;
    if (c.nwaves < 1) c.nwaves = 1;
    if (c.lds == 2) c.nwaves = nwork * kWavesPerGroup;   // one workgroup (of kClTrChannels threads) per item
    // Whole tiles of whole channel vectors take the straight-line path when all of
    // their loads can be vectors; then two row batches are in flight per lane.
    const bool straight = P.vector && c.vec_par && tile % kClUnroll == 0 &&
                          (!a->initial_states || c.vec_init) && (!a->seq_idx || c.vec_seq);
    P.unroll = straight ? (c.lds ? tile : 2 * kClUnroll) : kClUnroll;
    P.span = tile;
    P.channels_per_item = c.lds == 2 ? kClTrChannels : 64 * V;
    if (c.lds == 2) P.unroll = tile;
  }
  const int64_t waves = path == CCV_PATH_CHANNEL_FIRST ? plan->cf.nwaves : plan->cl.nwaves;
  const int64_t grid = (waves + kWavesPerGroup - 1) / kWavesPerGroup + tail_groups;
  if (grid > INT32_MAX) return CCV_E_SHAPE;
  m.nwork = nwork;
  m.xcd_q = (uint32_t)(grid / 8);
  m.xcd_r = (uint32_t)(grid % 8);
  P.grid = grid;
  P.work_items = nwork;
  plan->cf.m = m;
  plan->cl.m = m;
  return CCV_OK;
}

}  // namespace

extern "C" {

int ccv_fwd_check(const ccv_fwd_args_t* args) {
  Plan p;
  return validate(args, &p, last_cu_count());
}

// Plans touch no device: they size the grid for the GPU of the latest launch
// (256 CUs before any).
int ccv_fwd_plan(const ccv_fwd_args_t* args, ccv_plan_t* out) {
  Plan p;
  const int st = validate(args, &p, last_cu_count());
  if (st == CCV_OK && out) *out = p.pub;
  return st;
}

int ccv_fwd(const ccv_fwd_args_t* args, void* hip_stream) {
  // The grid is sized for the stream's own GPU; a validation error still comes
  // first when the runtime cannot name that GPU.
  const int cus = device_cu_count(hip_stream);
  Plan p;
  const int st = validate(args, &p, cus);
  if (st != CCV_OK) return st;
  if (p.pub.path == CCV_PATH_NONE || p.pub.grid == 0) return CCV_OK;
  if (cus < 0) return CCV_E_HIP;
  int err;
  if (p.pub.path == CCV_PATH_CHANNEL_FIRST)
    err = launch_cf(p.cf, args->x_dtype, args->K, p.silu, p.seq, p.pub.vector != 0,
                    (uint32_t)p.pub.grid, hip_stream);
  else
    err = launch_cl(p.cl, args->x_dtype, args->K, p.silu, p.seq, p.pub.vector != 0,
                    (uint32_t)p.pub.grid, hip_stream);
  return err == 0 ? CCV_OK : CCV_E_HIP;
}

const char* ccv_status_str(int s) {
  switch (s) {
    case CCV_OK: return "CCV_OK";
    case CCV_E_NULL: return "CCV_E_NULL";
    case CCV_E_SHAPE: return "CCV_E_SHAPE";
    case CCV_E_KSIZE: return "CCV_E_KSIZE";
    case CCV_E_DTYPE: return "CCV_E_DTYPE";
    case CCV_E_LAYOUT: return "CCV_E_LAYOUT";
    case CCV_E_UNSUPPORTED: return "CCV_E_UNSUPPORTED";
    case CCV_E_ALIAS: return "CCV_E_ALIAS";
    case CCV_E_HIP: return "CCV_E_HIP";
    case CCV_E_INTERNAL: return "CCV_E_INTERNAL";
    case CCV_E_ABI: return "CCV_E_ABI";
    case CCV_E_SCRATCH: return "CCV_E_SCRATCH";
  }
  return "CCV_E_UNKNOWN";
}

int ccv_abi_version(void) { return CCV_ABI_VERSION; }

}  // extern "C"
