// ccv_update_api.cpp -- C ABI of the update (decode) call: argument checks and
// the single kernel launch.  The operation and its contract are stated in ccv.h
// beside ccv_update; the checks mirror ccv_fwd's (K in {2,3,4}, three storage
// dtypes for x and weight, bias in the weight dtype, the state in x's dtype:
// Ch.4 "Dao interface and source map", section "Concrete limits of v1.5.0"),
// plus what an in-place update needs: the state and out layouts may not map two
// logical elements to one address, and no two of x, state, out may coincide.
//
// Nothing here touches a device except ccv_update's kernel launch.
#include <stdint.h>
#include <stdlib.h>

#include "ccv.h"
#include "ccv_checks.hpp"
#include "ccv_update_launch.hpp"

namespace {

using namespace ccv;
using namespace ccv::checks;

// Whether the 16-byte path of the kernel applies (see launch_update).
bool vector_path(const ccv_update_args_t* a) {
  const int es = elt_size(a->x_dtype);
  const int V = 16 / es;
  const int64_t B = a->B, C = a->C, L = a->L, H = a->K - 1;
  if (getenv("CCV_FORCE_SCALAR") && atoi(getenv("CCV_FORCE_SCALAR")) != 0) return false;
  if (C % V != 0) return false;
  if (!aligned16(a->weight) || (a->bias && !aligned16(a->bias))) return false;
  const bool x_ok = (a->x_stride[1] == 1 || C <= 1) && aligned16(a->x) &&
                    stride_ok16(B, a->x_stride[0], es) && stride_ok16(L, a->x_stride[2], es);
  const bool o_ok = (a->out_stride[1] == 1 || C <= 1) && aligned16(a->out) &&
                    stride_ok16(B, a->out_stride[0], es) && stride_ok16(L, a->out_stride[2], es);
  const bool s_ok = a->state_stride[2] == 1 && (a->state_stride[1] == H || C <= 1) &&
                    aligned16(a->state) && stride_ok16(B, a->state_stride[0], es);
  return x_ok && o_ok && s_ok;
}

int validate(const ccv_update_args_t* a, UpdArgs* u, uint32_t* grid, bool* vec) {
  if (!a) return CCV_E_NULL;
  if (a->struct_size != (int64_t)sizeof(ccv_update_args_t)) return CCV_E_ABI;
  if (a->B < 0 || a->C < 0 || a->L < 0) return CCV_E_SHAPE;
  if (a->K < 2 || a->K > 4) return CCV_E_KSIZE;
  if (a->x_dtype < 0 || a->x_dtype > 2 || a->w_dtype < 0 || a->w_dtype > 2) return CCV_E_DTYPE;
  if (a->activation != CCV_ACT_NONE && a->activation != CCV_ACT_SILU) return CCV_E_UNSUPPORTED;
  for (int d = 0; d < 3; ++d)
    if (a->x_stride[d] < 0 || a->out_stride[d] < 0 || a->state_stride[d] < 0) return CCV_E_LAYOUT;

  const int64_t B = a->B, C = a->C, L = a->L;
  const int K = a->K;
  *grid = 0;
  int64_t rows;
  if (__builtin_mul_overflow(B, C, &rows)) return CCV_E_SHAPE;
  if (rows == 0 || L == 0) return CCV_OK;        // nothing to compute; the state stays as it is

  if (!a->x || !a->weight || !a->state || !a->out) return CCV_E_NULL;
  if (a->out == a->x || a->state == a->x || a->state == a->out) return CCV_E_ALIAS;

  const int es = elt_size(a->x_dtype);
  const int64_t nx[3] = {B, C, L}, ns[3] = {B, C, K - 1};
  if (!fits_bytes(max_offset(nx, a->x_stride), es)) return CCV_E_SHAPE;
  if (!fits_bytes(max_offset(nx, a->out_stride), es)) return CCV_E_SHAPE;
  if (!fits_bytes(max_offset(ns, a->state_stride), es)) return CCV_E_SHAPE;
  if (!non_overlapping(nx, a->out_stride) || !non_overlapping(ns, a->state_stride)) return CCV_E_LAYOUT;

  *vec = vector_path(a);
  const int64_t per_group = (int64_t)kUpdateBlock * (*vec ? 16 / es : kUpdateRowsPerLane);
  const int64_t g = (rows + per_group - 1) / per_group;
  if (g > INT32_MAX) return CCV_E_SHAPE;

  *u = UpdArgs{};
  u->x = a->x;
  u->out = a->out;
  u->w = a->weight;
  u->bias = a->bias;
  u->state = a->state;
  u->C = C;
  u->L = L;
  u->rows = rows;
  u->x_sb = a->x_stride[0];
  u->x_sc = a->x_stride[1];
  u->x_sl = a->x_stride[2];
  u->o_sb = a->out_stride[0];
  u->o_sc = a->out_stride[1];
  u->o_sl = a->out_stride[2];
  u->s_sb = a->state_stride[0];
  u->s_sc = a->state_stride[1];
  u->s_si = a->state_stride[2];
  u->w_dtype = a->w_dtype;
  *grid = (uint32_t)g;
  return CCV_OK;
}

}  // namespace

extern "C" {

int ccv_update_check(const ccv_update_args_t* args) {
  UpdArgs u;
  uint32_t grid;
  bool vec;
  return validate(args, &u, &grid, &vec);
}

int ccv_update_plan(const ccv_update_args_t* args, ccv_plan_t* plan) {
  UpdArgs u;
  uint32_t grid;
  bool vec = false;
  const int st = validate(args, &u, &grid, &vec);
  if (st != CCV_OK || !plan) return st;
  *plan = ccv_plan_t{};
  plan->path = grid ? CCV_PATH_UPDATE : CCV_PATH_NONE;
  if (!grid) return st;
  const int rows_per_lane = vec ? 16 / elt_size(args->x_dtype) : kUpdateRowsPerLane;
  plan->vector = vec ? 1 : 0;
  plan->elems_per_lane = rows_per_lane;
  plan->unroll = 1;
  plan->grid = grid;
  plan->block = kUpdateBlock;
  plan->waves_per_group = kUpdateBlock / 64;
  plan->work_items = args->B * args->C;
  plan->span = args->L;
  plan->channels_per_item = rows_per_lane;
  return st;
}

int ccv_update(const ccv_update_args_t* args, void* hip_stream) {
  UpdArgs u;
  uint32_t grid;
  bool vec = false;
  const int st = validate(args, &u, &grid, &vec);
  if (st != CCV_OK) return st;
  if (grid == 0) return CCV_OK;
  const int err = launch_update(u, args->x_dtype, args->K, args->activation == CCV_ACT_SILU, vec, grid,
                                hip_stream);
  return err == 0 ? CCV_OK : CCV_E_HIP;
}

}  // extern "C"
