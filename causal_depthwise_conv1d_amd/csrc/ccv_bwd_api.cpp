// ccv_bwd_api.cpp -- C ABI of the backward: argument checks, the workspace size,
// and the two launches (gradient kernel, then the fixed-order reduction of the
// parameter gradients).  The operation and its contract are stated in ccv.h
// beside ccv_bwd; the checks mirror ccv_fwd's (K in {2,3,4}, three storage
// dtypes, bias in the weight dtype, states in x's dtype: Ch.4 "Dao interface
// and source map", section "Concrete limits of v1.5.0"), plus what the written
// gradients need: no aliasing with the inputs and no self-overlapping layouts.
//
// Nothing here touches a device except ccv_bwd's two kernel launches.
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>

#include "ccv.h"
#include "ccv_bwd_launch.hpp"
#include "ccv_checks.hpp"

namespace {

using namespace ccv;
using namespace ccv::checks;

struct BwdPlan {
  BwdArgs a;
  BwdReduceArgs r;
  int path = kBwdPathElement;
  int64_t grid = 0, rgrid = 0, ws_bytes = 0, items = 0;
};

// Which gradient kernel applies (see kBwdPath* in ccv_bwd_launch.hpp).
int choose_path(const ccv_bwd_args_t* a) {
  const char* force = getenv("CCV_FORCE_SCALAR");
  if (force && atoi(force) != 0) return kBwdPathElement;
  const int es = elt_size(a->x_dtype);
  const int V = 16 / es;
  const int64_t B = a->B, C = a->C, L = a->L;
  const bool aligned = aligned16(a->x) && aligned16(a->dout) && aligned16(a->dx);
  const int64_t* st[3] = {a->x_stride, a->dout_stride, a->dx_stride};
  // Channel-first rows of any length and offset take the register path (16-byte
  // accesses at any element alignment; the vector that straddles L moves element
  // by element).  The LDS-staged kernels need 16-byte aligned rows.
  // Channel-last step rows that are not 16-byte aligned (C not a multiple of V, or
  // an offset channel view) take the LDS-staged channel-last kernel's own variant.
  bool cf = true, cf16 = aligned && L % V == 0, cl = true, cl16 = aligned && C % V == 0;
  for (const int64_t* s : st) {
    cf = cf && s[2] == 1;
    cf16 = cf16 && s[2] == 1 && stride_ok16(B, s[0], es) && stride_ok16(C, s[1], es);
    cl = cl && s[1] == 1;
    cl16 = cl16 && s[1] == 1 && stride_ok16(B, s[0], es) && stride_ok16(L, s[2], es);
  }
  // The register path reads a lane's ids as 16-byte vectors beside its x; ids that
  // are not 16-byte aligned go through the LDS-staged kernel.
  if (cf && a->seq_idx && !aligned16(a->seq_idx)) return cf16 ? kBwdPathLdsCf : kBwdPathElement;
  if (cf) return cf16 ? kBwdPathRegCf : kBwdPathRegCfOdd;
  if (cl) return cl16 ? kBwdPathLdsCl : kBwdPathLdsClOdd;
  return kBwdPathElement;
}

// Checks every argument and fills *p; the workspace fields are checked only when
// `check_workspace` (ccv_bwd_workspace_size asks before there is one).
int validate(const ccv_bwd_args_t* a, BwdPlan* p, bool check_workspace = true) {
  if (!a) return CCV_E_NULL;
  if (a->struct_size != (int64_t)sizeof(ccv_bwd_args_t)) return CCV_E_ABI;
  if (a->B < 0 || a->C < 0 || a->L < 0) return CCV_E_SHAPE;
  if (a->K < 2 || a->K > 4) return CCV_E_KSIZE;
  if (a->x_dtype < 0 || a->x_dtype > 2 || a->w_dtype < 0 || a->w_dtype > 2) return CCV_E_DTYPE;
  if (a->activation != CCV_ACT_NONE && a->activation != CCV_ACT_SILU) return CCV_E_UNSUPPORTED;
  if (a->dinitial_states && !a->initial_states) return CCV_E_UNSUPPORTED;
  for (int d = 0; d < 3; ++d) {
    if (a->x_stride[d] < 0 || a->dout_stride[d] < 0 || a->dx_stride[d] < 0) return CCV_E_LAYOUT;
    if (a->initial_states && a->init_stride[d] < 0) return CCV_E_LAYOUT;
    if (a->dfinal_states && a->dfinal_stride[d] < 0) return CCV_E_LAYOUT;
    if (a->dinitial_states && a->dinit_stride[d] < 0) return CCV_E_LAYOUT;
  }

  const int64_t B = a->B, C = a->C, L = a->L;
  const int K = a->K;
  const int64_t H = K - 1;
  *p = BwdPlan{};
  if (C == 0) return CCV_OK;                      // no channel: nothing to write
  if (!a->weight || !a->dweight) return CCV_E_NULL;
  const bool rows = B > 0 && L > 0;
  if (rows && (!a->x || !a->dout || !a->dx)) return CCV_E_NULL;
  if (rows && (a->dx == a->x || a->dx == a->dout)) return CCV_E_ALIAS;
  if (a->dinitial_states && (a->dinitial_states == a->initial_states || a->dinitial_states == a->dfinal_states))
    return CCV_E_ALIAS;
  if (a->dweight == a->weight || (a->dbias && (a->dbias == a->bias || a->dbias == a->dweight))) return CCV_E_ALIAS;

  const int es = elt_size(a->x_dtype);
  const int64_t nx[3] = {B, C, L}, ns[3] = {B, C, H};
  if (rows) {
    if (!fits_bytes(max_offset(nx, a->x_stride), es)) return CCV_E_SHAPE;
    if (!fits_bytes(max_offset(nx, a->dout_stride), es)) return CCV_E_SHAPE;
    if (!fits_bytes(max_offset(nx, a->dx_stride), es)) return CCV_E_SHAPE;
    if (!non_overlapping(nx, a->dx_stride)) return CCV_E_LAYOUT;
  }
  if (a->initial_states && !fits_bytes(max_offset(ns, a->init_stride), es)) return CCV_E_SHAPE;
  if (a->dfinal_states && !fits_bytes(max_offset(ns, a->dfinal_stride), es)) return CCV_E_SHAPE;
  if (a->dinitial_states) {
    if (!fits_bytes(max_offset(ns, a->dinit_stride), es)) return CCV_E_SHAPE;
    if (!non_overlapping(ns, a->dinit_stride)) return CCV_E_LAYOUT;
  }
  int64_t bl;
  if (a->seq_idx && __builtin_mul_overflow(B, L, &bl)) return CCV_E_SHAPE;

  // Tiles of T steps (a row with L = 0 still has one, which writes d(initial_states)
  // from dfinal_states), grouped tpi to a partial row: one lane per (b, group, c) on
  // the element path, one wave per (b, group, 64 channels) on the LDS paths.  The
  // register-only channel-first path: segments of its own span, one per partial row,
  // one wave per (b, c, segment).
  const int path = rows ? choose_path(a) : kBwdPathElement;
  const bool reg = path == kBwdPathRegCf || path == kBwdPathRegCfOdd;
  const int64_t T = reg ? bwd_reg_span(a->x_dtype) : bwd_tile_steps(a->x_dtype);
  const int64_t ntt = L > 0 ? (L + T - 1) / T : 1;
  const bool channel_unit = (a->x_stride[1] == 1 || C <= 1) && !(a->x_stride[2] == 1 && L > 1);
  const int64_t tpi = channel_unit && !reg ? kBwdTilesPerItem : 1;
  const int64_t ngr = (ntt + tpi - 1) / tpi;
  int64_t nparts, lanes, ws;
  if (__builtin_mul_overflow(B, ngr, &nparts) || __builtin_mul_overflow(nparts, C, &lanes) ||
      __builtin_mul_overflow(nparts + bwd_reduce_rows(nparts), (int64_t)(K + 1) * C * 4, &ws))
    return CCV_E_SHAPE;
  const int64_t waves_per_group = kBwdBlock / 64;
  int64_t items, grid;
  if (path == kBwdPathElement) {
    items = lanes;
    grid = (lanes + kBwdBlock - 1) / kBwdBlock;
  } else if (reg) {
    items = lanes;                                  // B * C * segments, one wave each
    grid = (items + waves_per_group - 1) / waves_per_group;
  } else {
    items = nparts * ((C + 63) / 64);
    grid = items;
  }
  // Reduction launches: level kernels while more rows are left than the final kernel
  // takes (the first is the largest), then the final kernel, 64 columns per workgroup
  // (it also runs for B = 0, to write zeros).
  const int64_t width = (int64_t)(K + 1) * C;
  const int64_t rgrid = nparts > (int64_t)kBwdFanIn * kBwdFinalWaves
                            ? ((nparts + kBwdFanIn - 1) / kBwdFanIn * width + kBwdBlock - 1) / kBwdBlock
                            : (width + 63) / 64;
  if (grid > INT32_MAX || rgrid > INT32_MAX) return CCV_E_SHAPE;
  if (check_workspace && ws > 0) {
    if (!a->workspace) return CCV_E_NULL;
    if (a->workspace_bytes < ws) return CCV_E_SHAPE;
    if (!aligned16(a->workspace)) return CCV_E_LAYOUT;
  }

  BwdArgs& g = p->a;
  g.x = a->x;
  g.w = a->weight;
  g.bias = a->bias;
  g.seq = a->seq_idx;
  g.init = a->initial_states;
  g.dout = a->dout;
  g.dfs = a->dfinal_states;
  g.dx = a->dx;
  g.dinit = a->dinitial_states;
  g.part = static_cast<float*>(a->workspace);
  g.B = B;
  g.C = C;
  g.L = L;
  g.x_sb = a->x_stride[0];
  g.x_sc = a->x_stride[1];
  g.x_sl = a->x_stride[2];
  g.d_sb = a->dout_stride[0];
  g.d_sc = a->dout_stride[1];
  g.d_sl = a->dout_stride[2];
  g.g_sb = a->dx_stride[0];
  g.g_sc = a->dx_stride[1];
  g.g_sl = a->dx_stride[2];
  g.is_b = a->init_stride[0];
  g.is_c = a->init_stride[1];
  g.is_i = a->init_stride[2];
  g.fs_b = a->dfinal_stride[0];
  g.fs_c = a->dfinal_stride[1];
  g.fs_i = a->dfinal_stride[2];
  g.di_b = a->dinit_stride[0];
  g.di_c = a->dinit_stride[1];
  g.di_i = a->dinit_stride[2];
  g.T = T;
  g.ntt = ntt;
  g.tpi = tpi;
  g.ngr = ngr;
  g.lanes = lanes;
  g.items = items;
  g.w_dtype = a->w_dtype;
  g.off24 = std::max({a->x_stride[1], a->dout_stride[1], a->dx_stride[1]}) < (int64_t)(1 << 24) / es;

  BwdReduceArgs& r = p->r;
  r.in = g.part;
  r.dw = a->dweight;
  r.db = a->dbias;
  r.C = C;
  r.n_in = nparts;
  r.K = K;
  r.w_dtype = a->w_dtype;

  p->path = path;
  p->items = items;
  p->grid = grid;
  p->rgrid = rgrid;
  p->ws_bytes = ws;
  return CCV_OK;
}

}  // namespace

extern "C" {

int64_t ccv_bwd_workspace_size(const ccv_bwd_args_t* args) {
  BwdPlan p;
  const int st = validate(args, &p, false);
  return st == CCV_OK ? p.ws_bytes : st;
}

int ccv_bwd_check(const ccv_bwd_args_t* args) {
  BwdPlan p;
  return validate(args, &p);
}

int ccv_bwd_plan(const ccv_bwd_args_t* args, ccv_plan_t* plan) {
  BwdPlan p;
  const int st = validate(args, &p, false);      // a plan is wanted before the workspace exists
  if (st != CCV_OK || !plan) return st;
  *plan = ccv_plan_t{};
  const bool lds = p.path == kBwdPathLdsCf || p.path == kBwdPathLdsCl || p.path == kBwdPathLdsClOdd;
  plan->path = p.grid || p.rgrid ? CCV_PATH_BACKWARD : CCV_PATH_NONE;
  const bool reg = p.path == kBwdPathRegCf || p.path == kBwdPathRegCfOdd;
  plan->vector = reg ? kBwdPathRegCf : p.path == kBwdPathLdsClOdd ? kBwdPathLdsCl : p.path;
  plan->elems_per_lane = reg ? 16 / elt_size(args->x_dtype) : 1;
  plan->unroll = (int32_t)p.a.tpi;
  plan->grid = p.grid;
  plan->block = lds ? 64 : kBwdBlock;
  plan->waves_per_group = lds ? 1 : kBwdBlock / 64;
  plan->work_items = p.items;
  plan->span = p.a.T;
  plan->channels_per_item = lds ? 64 : 1;
  return st;
}

int ccv_bwd(const ccv_bwd_args_t* args, void* hip_stream) {
  BwdPlan p;
  const int st = validate(args, &p);
  if (st != CCV_OK) return st;
  if (p.grid > 0) {
    const int err = launch_bwd(p.a, args->x_dtype, args->K, args->activation == CCV_ACT_SILU,
                               args->seq_idx != nullptr, p.path, (uint32_t)p.grid, hip_stream);
    if (err != 0) return CCV_E_HIP;
  }
  if (p.rgrid > 0) {
    // Levels of the reduction tree, each reading the previous level's rows, then the
    // final kernel for the last two levels.
    BwdReduceArgs r = p.r;
    const int64_t width = (int64_t)(args->K + 1) * args->C;
    float* next = p.a.part ? p.a.part + p.r.n_in * width : nullptr;
    while (r.n_in > (int64_t)kBwdFanIn * kBwdFinalWaves) {
      const int64_t groups = (r.n_in + kBwdFanIn - 1) / kBwdFanIn;
      r.out = next;
      const int64_t grid = (groups * width + kBwdBlock - 1) / kBwdBlock;
      if (launch_bwd_reduce(r, (uint32_t)grid, hip_stream) != 0) return CCV_E_HIP;
      r.in = next;
      r.n_in = groups;
      next += groups * width;
    }
    const int waves = r.n_in > 0 ? (int)((r.n_in + kBwdFanIn - 1) / kBwdFanIn) : 1;
    const int64_t grid = (width + 63) / 64;
    if (launch_bwd_reduce_final(r, (uint32_t)grid, waves, hip_stream) != 0) return CCV_E_HIP;
  }
  return CCV_OK;
}

}  // extern "C"
