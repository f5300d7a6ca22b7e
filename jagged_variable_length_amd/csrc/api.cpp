// C ABI of libjattn.so: validation, planning, workspace layout and launches.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <initializer_list>
#include <new>
#include <string>
#include <vector>

#include "../../include/jattn.h"
#include "kernels.hpp"
#include "planner.hpp"

using jattn::KernelSel;
using jattn::UnitList;

struct jattn_plan {
  jattn_desc desc;
  float scale = 0.f;
  int B = 0, H = 0, D = 0;
  int64_t Tq = 0, Tk = 0, bias_elems = 0;
  double pairs = 0.0;  // allowed (i, j) pairs summed over samples (per head)
  int fwd_wq = 4, dq_wq = 4, dkdv_wkv = 4;
  int win_l = -1, win_r = -1;  // sliding window sides (clamped), -1 without one
  UnitList fwd, dkdv, dq, block;
  std::vector<int32_t> image;  // uploaded plan (int32 words)
  int64_t off_samples = 0, off_fwd_u = 0, off_fwd_o = 0, off_dkdv_u = 0, off_dkdv_o = 0;
  int64_t off_dq_u = 0, off_dq_o = 0, off_blk_u = 0, off_blk_o = 0;  // in int32 words
  int64_t off_theta = -1;  // RoPE theta table (fp64), in int32 words; -1 without RoPE
  // MXFP8: 32-row block tables (first row, rows) of the query and key rows
  bool mx = false;
  int64_t rb_q = 0, rb_k = 0, off_qblk = -1, off_kblk = -1;
  int64_t plan_bytes = 0, di_off = 0, lse2_off = 0, workspace_bytes = 0;
};

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int ok() {
  g_last_error.clear();
  return JATTN_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int kDefaultWorkers = 256;  // one persistent workgroup per CU

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Append a unit list to the image, 16-byte aligned sections.
void append(std::vector<int32_t>& img, const UnitList& L, int64_t* off_u, int64_t* off_o) {
  img.resize((size_t)align_up((int64_t)img.size(), 4), 0);
  *off_u = (int64_t)img.size();
  img.insert(img.end(), L.units.begin(), L.units.end());
  img.resize((size_t)align_up((int64_t)img.size(), 4), 0);
  *off_o = (int64_t)img.size();
  img.insert(img.end(), L.offsets.begin(), L.offsets.end());
}

int elem_size(int dt) { return dt == JATTN_F32 ? 4 : 2; }

KernelSel base_sel(const jattn_plan* p) {
  KernelSel k{};
  k.D = p->D;
  k.act = p->desc.act;
  k.bias = p->desc.has_bias != 0;
  k.dbias = p->desc.want_dbias != 0;
  k.dbias_f32 = p->desc.dbias_dtype == JATTN_F32;
  k.split = p->desc.split_operands != 0;
  k.in_f32 = p->desc.in_dtype == JATTN_F32;
  k.window = p->desc.mask == JATTN_MASK_WINDOW;
  return k;
}

const int32_t* ws_ptr(void* ws, int64_t off_words) {
  return reinterpret_cast<const int32_t*>(static_cast<char*>(ws) + off_words * 4);
}

int hip_fail(hipError_t e, const char* what) {
  return fail(JATTN_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int bwd_run(const jattn_plan* p, int32_t stages, const void* q, const void* k, const void* v, const void* bias,
            const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv, void* dbias,
            void* workspace, void* stream, bool fixed_scratch);

}  // namespace

extern "C" {

const char* jattn_strerror(int status) {
  switch (status) {
    case JATTN_OK: return "ok";
    case JATTN_E_NULL: return "null pointer";
    case JATTN_E_OFFSETS: return "invalid offsets";
    case JATTN_E_SHAPE: return "invalid shape";
    case JATTN_E_UNSUPPORTED: return "unsupported combination";
    case JATTN_E_ALIGN: return "misaligned pointer";
    case JATTN_E_WORKSPACE: return "workspace missing or too small";
    case JATTN_E_STATE: return "missing state";
    case JATTN_E_HIP: return "HIP runtime error";
    case JATTN_E_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

const char* jattn_last_error(void) { return g_last_error.c_str(); }

int jattn_plan_create(const jattn_desc* desc, const int64_t* q_offsets, const int64_t* kv_offsets,
                      jattn_plan** out) {
  if (!desc || !q_offsets || !kv_offsets || !out) return fail(JATTN_E_NULL, "null argument to jattn_plan_create");
  *out = nullptr;
  const jattn_desc& d = *desc;
  if (d.B < 0) return fail(JATTN_E_SHAPE, "B must be >= 0");
  if (d.H < 1 || d.H > 4096) return fail(JATTN_E_SHAPE, "H must be in [1, 4096]");
  if (d.D != 32 && d.D != 64 && d.D != 128) return fail(JATTN_E_SHAPE, "D must be 32, 64 or 128");
  if (d.act < JATTN_SOFTMAX || d.act > JATTN_GELU_POLY) return fail(JATTN_E_UNSUPPORTED, "unknown activation");
  if (d.act == JATTN_GELU_POLY && d.in_dtype != JATTN_BF16)
    return fail(JATTN_E_UNSUPPORTED, "the polynomial GELU needs bf16 inputs");
  if (d.mask != JATTN_MASK_NONE && d.mask != JATTN_MASK_BLOCKDIAG64 && d.mask != JATTN_MASK_WINDOW)
    return fail(JATTN_E_UNSUPPORTED, "unknown mask");
  if (d.mask == JATTN_MASK_WINDOW) {
    if (d.window_left < 0 || d.window_right < 0) return fail(JATTN_E_ARG, "window sides must be >= 0");
    if (d.in_dtype != JATTN_BF16) return fail(JATTN_E_UNSUPPORTED, "sliding-window mode needs bf16 inputs");
    if (d.want_dbias)
      return fail(JATTN_E_UNSUPPORTED, "sliding-window mode does not produce dbias (dense [H, lq, lk] layout)");
  }
  if (d.in_dtype != JATTN_BF16 && d.in_dtype != JATTN_F32 && d.in_dtype != JATTN_MXFP8)
    return fail(JATTN_E_UNSUPPORTED, "unknown in_dtype");
  if (d.in_dtype == JATTN_MXFP8) {
    if (d.D != 64 && d.D != 128) return fail(JATTN_E_UNSUPPORTED, "MXFP8 attention supports D = 64 or 128");
    if (d.mask != JATTN_MASK_NONE) return fail(JATTN_E_UNSUPPORTED, "MXFP8 attention has no block or window mask");
    if (d.has_bias) return fail(JATTN_E_UNSUPPORTED, "MXFP8 attention takes no bias");
    if (d.act == JATTN_GELU_POLY) return fail(JATTN_E_UNSUPPORTED, "MXFP8 attention: softmax, erf-GELU or SiLU");
  }
  if (d.out_dtype != JATTN_BF16 && d.out_dtype != JATTN_F32) return fail(JATTN_E_UNSUPPORTED, "unknown out_dtype");
  if (d.grad_dtype != JATTN_BF16 && d.grad_dtype != JATTN_F32) return fail(JATTN_E_UNSUPPORTED, "unknown grad_dtype");
  if (d.dbias_dtype != JATTN_BF16 && d.dbias_dtype != JATTN_F32) return fail(JATTN_E_UNSUPPORTED, "unknown dbias_dtype");
  if (d.in_dtype == JATTN_F32 && (d.out_dtype != JATTN_F32 || d.grad_dtype != JATTN_F32))
    return fail(JATTN_E_UNSUPPORTED, "fp32 inputs need fp32 outputs and gradients");
  if (d.in_dtype == JATTN_F32 && d.D > 64) return fail(JATTN_E_UNSUPPORTED, "fp32 inputs support D <= 64");
  if (d.want_dbias && !d.has_bias) return fail(JATTN_E_ARG, "want_dbias needs has_bias");
  if (d.has_bias != 0 && d.has_bias != 1) return fail(JATTN_E_ARG, "has_bias must be 0 or 1");
  if (d.mask == JATTN_MASK_BLOCKDIAG64 && (d.act != JATTN_SOFTMAX || d.has_bias))
    return fail(JATTN_E_UNSUPPORTED, "block-diagonal mode supports softmax without bias");
  if (d.mask == JATTN_MASK_BLOCKDIAG64 && d.in_dtype != JATTN_BF16)
    return fail(JATTN_E_UNSUPPORTED, "block-diagonal mode needs bf16 inputs");
  if (d.rope != 0 && d.rope != 1) return fail(JATTN_E_ARG, "rope must be 0 or 1");
  if (d.rope && d.mask != JATTN_MASK_BLOCKDIAG64)
    return fail(JATTN_E_UNSUPPORTED, "RoPE is fused into the block-diagonal kernels only");
  if (d.rope && !(d.rope_base <= 0.f || (d.rope_base > 1.f && !isinf(d.rope_base))))
    return fail(JATTN_E_ARG, "rope_base must be > 1 (or <= 0 for the default)");
  if (d.mask == JATTN_MASK_BLOCKDIAG64 && (d.num_workers % 2) != 0)
    return fail(JATTN_E_ARG, "block-diagonal mode needs an even num_workers (two per workgroup)");
  if (d.order < JATTN_HEAVY_FIRST || d.order > JATTN_LPT) return fail(JATTN_E_ARG, "unknown order");
  if (d.num_workers < 0 || d.num_workers > 65536) return fail(JATTN_E_ARG, "num_workers out of range");
  if (!(d.scale == d.scale) || isinf(d.scale)) return fail(JATTN_E_ARG, "scale must be finite");

  // offsets
  const int B = d.B;
  if (q_offsets[0] != 0 || kv_offsets[0] != 0) return fail(JATTN_E_OFFSETS, "offsets[0] must be 0");
  std::vector<int32_t> lq(B), lk(B);
  const int es = elem_size(d.in_dtype);
  // kernels address one sample's rows of any input, output or gradient with
  // 32-bit byte offsets, and mark lanes without a row by offsets >= 2^31
  const int es_max = std::max(es, std::max(elem_size(d.out_dtype), elem_size(d.grad_dtype)));
  const int64_t row_bytes = (int64_t)d.H * d.D * es_max;
  for (int b = 0; b < B; ++b) {
    const int64_t a = q_offsets[b + 1] - q_offsets[b];
    const int64_t c = kv_offsets[b + 1] - kv_offsets[b];
    if (a < 0 || c < 0) return fail(JATTN_E_OFFSETS, "offsets must be non-decreasing");
    if (q_offsets[b + 1] >= (int64_t(1) << 31) || kv_offsets[b + 1] >= (int64_t(1) << 31))
      return fail(JATTN_E_OFFSETS, "total rows must be < 2^31");
    if (a * row_bytes >= (int64_t(1) << 31) || c * row_bytes >= (int64_t(1) << 31))
      return fail(JATTN_E_SHAPE, "one sample must span < 2^31 bytes");
    if (d.has_bias && a * c * es >= (int64_t(1) << 30))
      return fail(JATTN_E_SHAPE, "one sample's bias block per head must span < 2^30 bytes");
    if (d.has_bias && d.want_dbias && a * c * elem_size(d.dbias_dtype) >= (int64_t(1) << 30))
      return fail(JATTN_E_SHAPE, "one sample's dbias block per head must span < 2^30 bytes");
    if (d.mask == JATTN_MASK_BLOCKDIAG64 && a != c)
      return fail(JATTN_E_SHAPE, "block-diagonal mode needs lq == lk for every sample");
    if (d.mask == JATTN_MASK_WINDOW && a != c)
      return fail(JATTN_E_SHAPE, "sliding-window mode needs lq == lk for every sample");
    lq[b] = (int32_t)a;
    lk[b] = (int32_t)c;
  }

  jattn_plan* p = new (std::nothrow) jattn_plan();
  if (!p) return fail(JATTN_E_ARG, "out of host memory");
  p->desc = d;
  p->B = B;
  p->H = d.H;
  p->D = d.D;
  p->scale = d.scale > 0.f ? d.scale : 1.0f / sqrtf((float)d.D);
  p->Tq = q_offsets[B];
  p->Tk = kv_offsets[B];
  if (d.mask == JATTN_MASK_WINDOW) {
    // a side longer than any sample is unbounded; the clamp keeps the
    // kernels' row +- side arithmetic inside int32 (rows < 2^25 per sample)
    p->win_l = std::min(d.window_left, 1 << 30);
    p->win_r = std::min(d.window_right, 1 << 30);
  }

  // sample table and algorithmic size
  p->image.assign((size_t)8 * B, 0);
  int64_t bias0 = 0;
  int64_t sum_lq = 0, n_q = 0, sum_lk = 0, n_k = 0;
  for (int b = 0; b < B; ++b) {
    int32_t* s = &p->image[(size_t)8 * b];
    s[0] = (int32_t)q_offsets[b];
    s[1] = lq[b];
    s[2] = (int32_t)kv_offsets[b];
    s[3] = lk[b];
    s[4] = (int32_t)(uint32_t)(bias0 & 0xffffffffLL);
    s[5] = (int32_t)(bias0 >> 32);
    if (d.in_dtype == JATTN_MXFP8) {
      // first 32-row block of the sample's queries / keys (MXFP8 scale and
      // transposed-code row blocks)
      s[6] = (int32_t)p->rb_q;
      s[7] = (int32_t)p->rb_k;
      p->rb_q += (lq[b] + 31) / 32;
      p->rb_k += (lk[b] + 31) / 32;
    }
    bias0 += (int64_t)d.H * lq[b] * lk[b];
    if (d.mask == JATTN_MASK_BLOCKDIAG64) {
      for (int s0 = 0; s0 < lq[b]; s0 += 64) {
        const double r = std::min(64, lq[b] - s0);
        p->pairs += r * r;
      }
    } else if (d.mask == JATTN_MASK_WINDOW) {
      // row i sees keys max(0, i - left) .. min(l - 1, i + right)
      int64_t n = 0;
      for (int64_t i = 0; i < lq[b]; ++i)
        n += std::min<int64_t>(lk[b] - 1, i + p->win_r) - std::max<int64_t>(0, i - p->win_l) + 1;
      p->pairs += (double)n;
    } else {
      p->pairs += (double)lq[b] * (double)lk[b];
    }
    if (lq[b] > 0) { sum_lq += lq[b]; ++n_q; }
    if (lk[b] > 0) { sum_lk += lk[b]; ++n_k; }
  }
  p->bias_elems = bias0;
  p->off_samples = 0;

  const int W = d.num_workers > 0 ? d.num_workers
                                  : (d.mask == JATTN_MASK_BLOCKDIAG64 ? 2 * kDefaultWorkers : kDefaultWorkers);
  const jattn::Order order = (jattn::Order)d.order;
  if (d.mask == JATTN_MASK_BLOCKDIAG64) {
    jattn::plan_units(jattn::kKindBlock, lq, lk, d.H, 64, 64, W, order, &p->block);
  } else if (d.in_dtype == JATTN_MXFP8) {
    // MXFP8 forward: 128-row query tiles (four waves of 32 rows), 64-key steps
    p->mx = true;
    p->fwd_wq = 4;
    jattn::plan_units(jattn::kKindFwd, lq, lk, d.H, 128, 64, W, order, &p->fwd);
    // backward: dK/dV over 128-key tiles with 64-query steps, dQ like the forward
    jattn::plan_units(jattn::kKindDkdv, lq, lk, d.H, 128, 64, W, order, &p->dkdv);
    jattn::plan_units(jattn::kKindDq, lq, lk, d.H, 128, 64, W, order, &p->dq);
  } else {
    // Query-tile shape: 4 waves x 32 rows, or (short queries) one 32-row
    // group whose key tiles are split over the 4 waves.
    p->fwd_wq = (n_q > 0 && sum_lq <= 48 * n_q) ? 1 : 4;
    // the bf16 short-query forward has no room for a bias tile at D = 128
    if (d.in_dtype == JATTN_BF16 && d.D == 128 && d.has_bias) p->fwd_wq = 4;
    p->dq_wq = (n_q > 0 && sum_lq <= 48 * n_q) ? 1 : 4;
    // nor has the bf16 short-query dQ kernel
    if (d.in_dtype == JATTN_BF16 && d.D == 128 && d.has_bias) p->dq_wq = 4;
    // bf16 long queries: 8 query groups of 32 rows over one 32-key block per
    // step (no key split, so no partials to combine); the windowed kernels
    // keep 4 query groups x 2 key halves (128-row tiles visit fewer keys
    // outside a window); fp32 inputs use 128-row tiles with 64-key steps
    if (d.in_dtype == JATTN_BF16) {
      if (p->fwd_wq == 4) p->fwd_wq = 8;
      if (p->dq_wq == 4) p->dq_wq = 8;
    }
    if (d.mask == JATTN_MASK_WINDOW) p->fwd_wq = p->dq_wq = 4;
    // bf16 forward at D <= 64 without a bias or window, long queries: 4 query
    // groups over one 32-key block per step, three workgroups per CU (the
    // kernel's ~160 registers fit three waves per SIMD), over three times the
    // workers (fwd2_waves_per_simd applies the same rule).  dQ keeps 8 x 1:
    // the same shape there measured slower (its K/V stages serve half the
    // query rows)
    const bool fwd_three = d.in_dtype == JATTN_BF16 && d.D <= 64 && !d.has_bias && d.mask == JATTN_MASK_NONE &&
                           p->fwd_wq == 8;
    if (fwd_three) p->fwd_wq = 4;
    // the same shape at D = 128 (softmax without a bias or window): two
    // workgroups per CU over twice the workers, each ~245 registers and 72 KB
    // of LDS; a barrier then spans four waves instead of eight
    const bool fwd_two = d.in_dtype == JATTN_BF16 && d.D == 128 && !d.has_bias && d.mask == JATTN_MASK_NONE &&
                         d.act == JATTN_SOFTMAX && p->fwd_wq == 8;
    if (fwd_two) p->fwd_wq = 4;
    // dQ at D = 128 (softmax without a bias, window or split operands): the
    // same 128-row tiles over 32-key steps, two workgroups per CU over twice
    // the workers; at D <= 64 (softmax without a bias or window, split
    // operands allowed) the same
    const bool dq_two = d.in_dtype == JATTN_BF16 && d.D == 128 && !d.has_bias && d.mask == JATTN_MASK_NONE &&
                        d.act == JATTN_SOFTMAX && !d.split_operands && p->dq_wq == 8;
    const bool dq_two64 = d.in_dtype == JATTN_BF16 && d.D <= 64 && !d.has_bias && d.mask == JATTN_MASK_NONE &&
                          d.act == JATTN_SOFTMAX && p->dq_wq == 8;
    if (dq_two || dq_two64) p->dq_wq = 4;
    auto step_of = [](int wq) { return wq == 8 ? 32 : wq == 4 ? 64 : 128; };
    const int fwd_tile = 32 * p->fwd_wq, fwd_step = (fwd_three || fwd_two) ? 32 : step_of(p->fwd_wq);
    const int dq_tile = 32 * p->dq_wq, dq_step = (dq_two || dq_two64) ? 32 : step_of(p->dq_wq);
    // Key-tile shape of dK/dV: 32, 64 or 128 keys per unit.
    p->dkdv_wkv = (n_k > 0 && sum_lk <= 32 * n_k) ? 1 : (n_k > 0 && sum_lk <= 64 * n_k) ? 2 : 4;
    // the bf16 dK/dV kernel keeps three or four step stages in LDS: 128-query
    // steps (32-key units) do not leave room for three at D = 128
    if (d.in_dtype == JATTN_BF16 && d.D == 128 && p->dkdv_wkv == 1) p->dkdv_wkv = 2;
    if (d.mask == JATTN_MASK_WINDOW) p->dkdv_wkv = 4;
    const int dkdv_tile = 32 * p->dkdv_wkv, dkdv_step = 32 * (4 / p->dkdv_wkv);
    jattn::Window win;
    win.left = p->win_l;
    win.right = p->win_r;
    jattn::plan_units(jattn::kKindFwd, lq, lk, d.H, fwd_tile, fwd_step, fwd_three ? 3 * W : fwd_two ? 2 * W : W, order, &p->fwd, win);
    jattn::plan_units(jattn::kKindDq, lq, lk, d.H, dq_tile, dq_step, (dq_two || dq_two64) ? 2 * W : W, order, &p->dq, win);
    // the bf16 dK/dV kernel runs two workgroups per CU at D <= 64 without a
    // bias or window on 64- or 128-key units (not with erf-GELU): twice the
    // workers (the kernel's dkdv2_waves_per_simd applies the same rule)
    const bool dkdv_two = d.in_dtype == JATTN_BF16 && d.D <= 64 && !d.has_bias && d.mask != JATTN_MASK_WINDOW &&
                          p->dkdv_wkv >= 2 && d.act != JATTN_GELU_ERF;
    jattn::plan_units(jattn::kKindDkdv, lq, lk, d.H, dkdv_tile, dkdv_step, dkdv_two ? 2 * W : W, order, &p->dkdv,
                      win);
  }
  append(p->image, p->fwd, &p->off_fwd_u, &p->off_fwd_o);
  append(p->image, p->dkdv, &p->off_dkdv_u, &p->off_dkdv_o);
  append(p->image, p->dq, &p->off_dq_u, &p->off_dq_o);
  append(p->image, p->block, &p->off_blk_u, &p->off_blk_o);
  if (d.rope) {
    // theta_j = base^(-2j/D), j < D/2, as fp64 words
    const double base = d.rope_base > 0.f ? (double)d.rope_base : 10000.0;
    p->image.resize((size_t)align_up((int64_t)p->image.size(), 4), 0);
    p->off_theta = (int64_t)p->image.size();
    for (int j = 0; j < d.D / 2; ++j) {
      const double th = pow(base, -2.0 * j / d.D);
      int32_t w[2];
      memcpy(w, &th, 8);
      p->image.push_back(w[0]);
      p->image.push_back(w[1]);
    }
  }
  if (p->mx) {
    // 32-row block tables of the quantiser: (first row, rows) per block
    auto blocks = [&](const int64_t* off, int64_t* at) {
      p->image.resize((size_t)align_up((int64_t)p->image.size(), 4), 0);
      *at = (int64_t)p->image.size();
      for (int b = 0; b < B; ++b)
        for (int64_t r = off[b]; r < off[b + 1]; r += 32) {
          p->image.push_back((int32_t)r);
          p->image.push_back((int32_t)std::min<int64_t>(32, off[b + 1] - r));
        }
    };
    blocks(q_offsets, &p->off_qblk);
    blocks(kv_offsets, &p->off_kblk);
  }
  p->plan_bytes = (int64_t)p->image.size() * 4;
  p->di_off = align_up(p->plan_bytes, 256);
  p->lse2_off = p->di_off + align_up(p->Tq * d.H * 4, 256);
  p->workspace_bytes = p->lse2_off + align_up(p->Tq * d.H * 4, 256);
  *out = p;
  return ok();
}

int jattn_plan_info(const jattn_plan* p, jattn_plan_summary* s) {
  if (!p || !s) return fail(JATTN_E_NULL, "null argument to jattn_plan_info");
  memset(s, 0, sizeof(*s));
  s->workspace_bytes = p->workspace_bytes;
  s->Tq = p->Tq;
  s->Tk = p->Tk;
  s->bias_elems = p->bias_elems;
  s->flops_fwd = 4.0 * p->H * p->D * p->pairs;
  s->flops_bwd = 2.5 * s->flops_fwd;
  auto fill = [](const UnitList& L, jattn_kernel_plan* k) {
    k->tile_rows = L.tile_rows;
    k->step_rows = L.step_rows;
    k->num_workers = L.num_workers;
    k->n_units = (int32_t)L.n_units();
  };
  fill(p->fwd, &s->fwd);
  fill(p->dkdv, &s->dkdv);
  fill(p->dq, &s->dq);
  fill(p->block, &s->block);
  return ok();
}

int jattn_plan_export(const jattn_plan* p, int32_t which, int32_t* dst, int64_t cap, int64_t* n) {
  if (!p || !n) return fail(JATTN_E_NULL, "null argument to jattn_plan_export");
  const UnitList* L = nullptr;
  switch (which / 2) {
    case JATTN_PLAN_FWD: L = &p->fwd; break;
    case JATTN_PLAN_DKDV: L = &p->dkdv; break;
    case JATTN_PLAN_DQ: L = &p->dq; break;
    case JATTN_PLAN_BLOCK: L = &p->block; break;
    default: return fail(JATTN_E_ARG, "unknown plan part");
  }
  if (which < 0 || which > 7) return fail(JATTN_E_ARG, "unknown plan part");
  const std::vector<int32_t>& v = (which % 2 == 0) ? L->units : L->offsets;
  *n = (int64_t)v.size();
  if (!dst) return ok();
  if (cap < (int64_t)v.size()) return fail(JATTN_E_ARG, "export buffer too small");
  if (!v.empty()) memcpy(dst, v.data(), v.size() * 4);
  return ok();
}

int jattn_plan_upload(const jattn_plan* p, void* workspace, int64_t workspace_bytes, void* stream) {
  if (!p) return fail(JATTN_E_NULL, "null plan");
  if (!workspace) return fail(JATTN_E_WORKSPACE, "null workspace");
  if (workspace_bytes < p->workspace_bytes) return fail(JATTN_E_WORKSPACE, "workspace too small");
  if (!aligned(workspace, 256)) return fail(JATTN_E_ALIGN, "workspace must be 256-byte aligned");
  if (p->plan_bytes == 0) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(workspace, p->image.data(), (size_t)p->plan_bytes, hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(plan)");
  // the source is pageable plan memory: wait so that the plan may be freed
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize(plan)");
  return ok();
}

int jattn_fwd(const jattn_plan* p, const void* q, const void* k, const void* v, const void* bias, void* o,
              float* lse, void* workspace, void* stream) {
  if (!p) return fail(JATTN_E_NULL, "null plan");
  if (p->mx) return fail(JATTN_E_UNSUPPORTED, "an MXFP8 plan runs through jattn_mx_fwd");
  if (p->Tq == 0) return ok();
  if (!q || !o || (p->Tk > 0 && (!k || !v))) return fail(JATTN_E_NULL, "null q/k/v/o");
  if (p->desc.has_bias && !bias && p->bias_elems > 0) return fail(JATTN_E_NULL, "bias required (has_bias = 1)");
  if (!workspace) return fail(JATTN_E_WORKSPACE, "null workspace");
  if (!aligned(workspace, 256)) return fail(JATTN_E_ALIGN, "workspace must be 256-byte aligned");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(JATTN_E_ALIGN, "q/k/v/o must be 16-byte aligned");
  const int es = elem_size(p->desc.in_dtype);
  if (bias && !aligned(bias, (uintptr_t)es)) return fail(JATTN_E_ALIGN, "bias must be element-aligned");
  if (lse && !aligned(lse, 4)) return fail(JATTN_E_ALIGN, "lse must be 4-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int32_t* samples = ws_ptr(workspace, p->off_samples);

  jattn::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.bias = p->desc.has_bias ? bias : nullptr;
  a.o = o;
  a.lse = (p->desc.act == JATTN_SOFTMAX) ? lse : nullptr;
  a.units = ws_ptr(workspace, p->off_fwd_u);
  a.worker_off = ws_ptr(workspace, p->off_fwd_o);
  a.samples = samples;
  a.H = p->H;
  a.scale = p->scale;
  a.scale_log2 = p->scale * 1.4426950408889634f;
  a.bias_elems = p->bias_elems;
  a.win_l = p->win_l;
  a.win_r = p->win_r;
  KernelSel sel = base_sel(p);
  sel.out_f32 = p->desc.out_dtype == JATTN_F32;
  sel.wq = p->fwd_wq;
  hipError_t e;
  if (p->desc.mask == JATTN_MASK_BLOCKDIAG64) {
    if (p->block.n_units() == 0) return ok();
    a.lse = nullptr;  // no row statistics leave a block
    a.units = ws_ptr(workspace, p->off_blk_u);
    a.worker_off = ws_ptr(workspace, p->off_blk_o);
    if (p->off_theta >= 0) a.rope_theta = reinterpret_cast<const double*>(ws_ptr(workspace, p->off_theta));
    e = jattn::launch_block_fwd(a, sel, p->block.num_workers / 2, st);
  } else {
    e = jattn::launch_fwd(a, sel, p->fwd.num_workers, st);
  }
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  return ok();
}

int jattn_bwd(const jattn_plan* p, const void* q, const void* k, const void* v, const void* bias, const void* o,
              const float* lse, const void* dout, void* dq, void* dk, void* dv, void* dbias, void* workspace,
              void* stream) {
  return jattn_bwd_stages(p, JATTN_BWD_ALL, q, k, v, bias, o, lse, dout, dq, dk, dv, dbias, workspace, stream);
}

int jattn_bwd_stages(const jattn_plan* p, int32_t stages, const void* q, const void* k, const void* v,
                     const void* bias, const void* o, const float* lse, const void* dout, void* dq, void* dk,
                     void* dv, void* dbias, void* workspace, void* stream) {
  return bwd_run(p, stages, q, k, v, bias, o, lse, dout, dq, dk, dv, dbias, workspace, stream, false);
}

int jattn_bwd_fixed_scratch(const jattn_plan* p, const void* q, const void* k, const void* v, const void* bias,
                            const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                            void* dbias, void* workspace, void* stream) {
  return bwd_run(p, JATTN_BWD_ALL, q, k, v, bias, o, lse, dout, dq, dk, dv, dbias, workspace, stream, true);
}

}  // extern "C"

namespace {

// Row-statistics region (Di, then LSE * log2 e, each Tq * H floats) of a
// backward: in the workspace after the plan, or at the start of the library's
// fixed device scratch.
int64_t rowstat_bytes(const jattn_plan* p) { return 2 * align_up(p->Tq * p->H * 4, 256); }

int bwd_run(const jattn_plan* p, int32_t stages, const void* q, const void* k, const void* v, const void* bias,
            const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv, void* dbias,
            void* workspace, void* stream, bool fixed_scratch) {
  if (!p) return fail(JATTN_E_NULL, "null plan");
  if (p->mx) return fail(JATTN_E_UNSUPPORTED, "an MXFP8 plan has no bf16 backward");
  if (stages < 0 || stages > JATTN_BWD_ALL) return fail(JATTN_E_ARG, "unknown backward stage mask");
  // softmax outside block mode keeps row statistics from the forward
  const bool softmax_dense = p->desc.act == JATTN_SOFTMAX && p->desc.mask != JATTN_MASK_BLOCKDIAG64;
  if (fixed_scratch && softmax_dense && rowstat_bytes(p) > (int64_t)jattn::fixed_scratch_bytes())
    return fail(JATTN_E_WORKSPACE, "the row statistics of this plan (" + std::to_string(rowstat_bytes(p)) +
                                       " bytes, Tq * H = " + std::to_string(p->Tq * p->H) +
                                       ") exceed the fixed scratch of " +
                                       std::to_string(jattn::fixed_scratch_bytes()) + " bytes");
  if (p->Tq == 0 && p->Tk == 0) return ok();
  if ((p->Tq > 0 && (!q || !dout || !dq)) || (p->Tk > 0 && (!k || !v || !dk || !dv)))
    return fail(JATTN_E_NULL, "null q/k/v/dout/dq/dk/dv");
  if (p->desc.has_bias && !bias && p->bias_elems > 0) return fail(JATTN_E_NULL, "bias required (has_bias = 1)");
  if (p->desc.want_dbias && !dbias && p->bias_elems > 0) return fail(JATTN_E_NULL, "dbias required (want_dbias = 1)");
  if (softmax_dense && p->Tq > 0 && (!o || !lse)) return fail(JATTN_E_STATE, "softmax backward needs o and lse");
  if (!workspace) return fail(JATTN_E_WORKSPACE, "null workspace");
  if (!aligned(workspace, 256)) return fail(JATTN_E_ALIGN, "workspace must be 256-byte aligned");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) || !aligned(dq, 16) ||
      !aligned(dk, 16) || !aligned(dv, 16) || !aligned(o, 16))
    return fail(JATTN_E_ALIGN, "value tensors must be 16-byte aligned");
  const int es = elem_size(p->desc.in_dtype);
  if ((bias && !aligned(bias, (uintptr_t)es)) || (dbias && !aligned(dbias, (uintptr_t)elem_size(p->desc.dbias_dtype))))
    return fail(JATTN_E_ALIGN, "bias/dbias must be element-aligned");
  if (lse && !aligned(lse, 4)) return fail(JATTN_E_ALIGN, "lse must be 4-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);

  float* di = reinterpret_cast<float*>(static_cast<char*>(workspace) + p->di_off);
  float* lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + p->lse2_off);
  if (fixed_scratch && softmax_dense && p->Tq > 0) {
    // the current device's copy of the fixed scratch; the stream must belong
    // to that device
    if (st != nullptr) {
      int sdev = -1, cdev = -1;
      hipError_t e = hipStreamGetDevice(st, &sdev);
      if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
      e = hipGetDevice(&cdev);
      if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
      if (sdev != cdev) return fail(JATTN_E_ARG, "the stream belongs to another device than the current one");
    }
    void* base = nullptr;
    const hipError_t e = jattn::fixed_scratch_address(&base);
    if (e != hipSuccess) return hip_fail(e, "fixed scratch address (hipGetSymbolAddress)");
    di = reinterpret_cast<float*>(base);
    lse2 = reinterpret_cast<float*>(static_cast<char*>(base) + align_up(p->Tq * p->H * 4, 256));
  }
  KernelSel sel = base_sel(p);
  sel.out_f32 = p->desc.grad_dtype == JATTN_F32;
  sel.wq = p->dq_wq;
  sel.wkv = p->dkdv_wkv;
  hipError_t e;
  if (p->desc.mask == JATTN_MASK_BLOCKDIAG64) {
    if (p->block.n_units() == 0 || !(stages & (JATTN_BWD_DKDV | JATTN_BWD_DQ))) return ok();
    jattn::BwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.dout = dout;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.units = ws_ptr(workspace, p->off_blk_u);
    a.worker_off = ws_ptr(workspace, p->off_blk_o);
    a.samples = ws_ptr(workspace, p->off_samples);
    if (p->off_theta >= 0) a.rope_theta = reinterpret_cast<const double*>(ws_ptr(workspace, p->off_theta));
    a.H = p->H;
    a.scale = p->scale;
    a.scale_log2 = p->scale * 1.4426950408889634f;
    e = jattn::launch_block_bwd(a, sel, p->block.num_workers, st);  // one wave pair per workgroup
    if (e != hipSuccess) return hip_fail(e, "block backward launch");
    return ok();
  }
  // bf16 softmax: the dQ pass forms Di and LSE*log2e itself from O, dO and
  // LSE and writes them for dK/dV, which then runs after it (not with fp32 O
  // at D = 128, whose registers do not fit beside dQ's other operands)
  const bool fold = softmax_dense && !sel.in_f32 && !(p->D == 128 && p->desc.out_dtype == JATTN_F32);
  sel.o_f32 = p->desc.out_dtype == JATTN_F32;
  sel.fold = fold;
  const bool dq_forms_rowstats = fold && (stages & JATTN_BWD_DQ);
  if (softmax_dense && p->Tq > 0 && (stages & JATTN_BWD_PREP) && !dq_forms_rowstats) {
    jattn::DiArgs da{o, dout, di, p->Tq * p->H, lse, lse2};
    e = jattn::launch_di(da, sel, p->desc.out_dtype == JATTN_F32, st);
    if (e != hipSuccess) return hip_fail(e, "Di launch");
  }
  jattn::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.bias = p->desc.has_bias ? bias : nullptr;
  a.dout = dout;
  a.lse = lse;
  a.di = di;
  a.lse2 = lse2;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dbias = p->desc.want_dbias ? dbias : nullptr;
  a.samples = ws_ptr(workspace, p->off_samples);
  a.H = p->H;
  a.scale = p->scale;
  a.scale_log2 = p->scale * 1.4426950408889634f;
  a.bias_elems = p->bias_elems;
  a.win_l = p->win_l;
  a.win_r = p->win_r;
  a.o = o;
  if (fold) {
    a.rs_di = di;
    a.rs_lse2 = lse2;
  }
  auto run_dkdv = [&]() -> int {
    if (p->dkdv.n_units() > 0 && (stages & JATTN_BWD_DKDV)) {
      a.units = ws_ptr(workspace, p->off_dkdv_u);
      a.worker_off = ws_ptr(workspace, p->off_dkdv_o);
      const hipError_t e2 = jattn::launch_dkdv(a, sel, p->dkdv.num_workers, st);
      if (e2 != hipSuccess) return hip_fail(e2, "dK/dV launch");
    }
    return JATTN_OK;
  };
  auto run_dq = [&]() -> int {
    if (p->dq.n_units() > 0 && (stages & JATTN_BWD_DQ)) {
      a.units = ws_ptr(workspace, p->off_dq_u);
      a.worker_off = ws_ptr(workspace, p->off_dq_o);
      const hipError_t e2 = jattn::launch_dq(a, sel, p->dq.num_workers, st);
      if (e2 != hipSuccess) return hip_fail(e2, "dQ launch");
    }
    return JATTN_OK;
  };
  // with the row statistics formed by dQ, dK/dV reads them after it
  const int r1 = fold ? run_dq() : run_dkdv();
  if (r1 != JATTN_OK) return r1;
  const int r2 = fold ? run_dkdv() : run_dq();
  if (r2 != JATTN_OK) return r2;
  return ok();
}

}  // namespace

extern "C" {

void jattn_plan_destroy(jattn_plan* p) { delete p; }

int jattn_mx_sizes(const jattn_plan* p, int32_t rows, int64_t* codes_bytes, int64_t* codes_t_bytes,
                   int64_t* scales_bytes) {
  if (!p || !codes_bytes || !codes_t_bytes || !scales_bytes) return fail(JATTN_E_NULL, "null argument");
  if (!p->mx) return fail(JATTN_E_UNSUPPORTED, "not an MXFP8 plan");
  if (rows != JATTN_MX_Q && rows != JATTN_MX_KV) return fail(JATTN_E_ARG, "rows must be JATTN_MX_Q or JATTN_MX_KV");
  const int64_t T = rows == JATTN_MX_Q ? p->Tq : p->Tk;
  const int64_t RB = rows == JATTN_MX_Q ? p->rb_q : p->rb_k;
  *codes_bytes = T * p->H * p->D;
  *codes_t_bytes = RB * p->H * p->D * 32;
  // rounded up to whole dwords: the kernels read scale bytes as aligned dwords
  *scales_bytes = align_up(RB * p->H * (p->D / 32), 4);
  return ok();
}

int jattn_mx_quantize(const jattn_plan* p, int32_t rows, const void* x, const jattn_mx_tensor* out, void* workspace,
                      void* stream) {
  if (!p || !out) return fail(JATTN_E_NULL, "null plan or output");
  if (!p->mx) return fail(JATTN_E_UNSUPPORTED, "not an MXFP8 plan");
  if (rows != JATTN_MX_Q && rows != JATTN_MX_KV) return fail(JATTN_E_ARG, "rows must be JATTN_MX_Q or JATTN_MX_KV");
  const int64_t T = rows == JATTN_MX_Q ? p->Tq : p->Tk;
  const int64_t RB = rows == JATTN_MX_Q ? p->rb_q : p->rb_k;
  if (T == 0) return ok();
  if (!x || !out->codes || !out->scales) return fail(JATTN_E_NULL, "null x / codes / scales");
  if (!workspace) return fail(JATTN_E_WORKSPACE, "null workspace");
  if (!aligned(workspace, 256)) return fail(JATTN_E_ALIGN, "workspace must be 256-byte aligned");
  if (!aligned(x, 16) || !aligned(out->codes, 16) || (out->codes_t && !aligned(out->codes_t, 16)))
    return fail(JATTN_E_ALIGN, "x / codes / codes_t must be 16-byte aligned");
  jattn::MxQuantArgs a{};
  a.x = x;
  a.codes = static_cast<uint8_t*>(out->codes);
  a.codes_t = static_cast<uint8_t*>(out->codes_t);
  a.scales = static_cast<uint8_t*>(out->scales);
  a.blocks = ws_ptr(workspace, rows == JATTN_MX_Q ? p->off_qblk : p->off_kblk);
  a.H = p->H;
  a.nblocks = RB;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = p->D == 128 ? jattn::launch_mx_quant_128(a, st) : jattn::launch_mx_quant_64(a, st);
  if (e != hipSuccess) return hip_fail(e, "MXFP8 quantisation launch");
  return ok();
}

int jattn_mx_bwd(const jattn_plan* p, int32_t stages, const jattn_mx_tensor* q, const jattn_mx_tensor* k,
                 const jattn_mx_tensor* v, const void* o, const float* lse, const jattn_mx_tensor* dout, void* dq,
                 void* dk, void* dv, void* workspace, void* stream) {
  if (!p) return fail(JATTN_E_NULL, "null plan");
  if (!p->mx) return fail(JATTN_E_UNSUPPORTED, "not an MXFP8 plan");
  if (stages < 0 || stages > JATTN_BWD_ALL) return fail(JATTN_E_ARG, "unknown backward stage mask");
  if (p->Tq == 0 && p->Tk == 0) return ok();
  const bool softmax = p->desc.act == JATTN_SOFTMAX;
  if (!q || !k || !v || !dout) return fail(JATTN_E_NULL, "null q / k / v / dout");
  if ((p->Tq > 0 && (!q->codes || !q->codes_t || !q->scales || !dout->codes || !dout->codes_t || !dout->scales ||
                     !dq)) ||
      (p->Tk > 0 && (!k->codes || !k->codes_t || !k->scales || !v->codes || !v->scales || !dk || !dv)))
    return fail(JATTN_E_NULL, "the backward reads q, dout (codes, codes_t, scales), k (codes, codes_t, scales), "
                              "v (codes, scales) and writes dq, dk, dv");
  if (softmax && p->Tq > 0 && (!o || !lse)) return fail(JATTN_E_STATE, "softmax backward needs o and lse");
  if (!workspace) return fail(JATTN_E_WORKSPACE, "null workspace");
  if (!aligned(workspace, 256)) return fail(JATTN_E_ALIGN, "workspace must be 256-byte aligned");
  for (const jattn_mx_tensor* t : {q, k, v, dout})
    if ((t->codes && !aligned(t->codes, 16)) || (t->codes_t && !aligned(t->codes_t, 16)) ||
        (t->scales && !aligned(t->scales, 4)))
      return fail(JATTN_E_ALIGN, "codes / codes_t must be 16-byte aligned, scales 4-byte aligned");
  if (!aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || (o && !aligned(o, 16)) || (lse && !aligned(lse, 4)))
    return fail(JATTN_E_ALIGN, "o / dq / dk / dv must be 16-byte aligned, lse 4-byte aligned");
  auto tens = [](const jattn_mx_tensor* t) {
    return jattn::MxTensor{static_cast<const uint8_t*>(t->codes), static_cast<const uint8_t*>(t->codes_t),
                           static_cast<const uint8_t*>(t->scales)};
  };
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* di = reinterpret_cast<float*>(static_cast<char*>(workspace) + p->di_off);
  float* lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + p->lse2_off);
  hipError_t e;
  if (softmax && p->Tq > 0 && (stages & JATTN_BWD_PREP)) {
    jattn::MxDiArgs da{};
    da.dout = tens(dout);
    da.o = o;
    da.lse = lse;
    da.di = di;
    da.lse2 = lse2;
    da.blocks = ws_ptr(workspace, p->off_qblk);
    da.H = p->H;
    da.nblocks = p->rb_q;
    const bool of32 = p->desc.out_dtype == JATTN_F32;
    e = p->D == 128 ? jattn::launch_mx_di_128(da, of32, st) : jattn::launch_mx_di_64(da, of32, st);
    if (e != hipSuccess) return hip_fail(e, "MXFP8 Di launch");
  }
  jattn::MxBwdArgs a{};
  a.q = tens(q);
  a.k = tens(k);
  a.v = tens(v);
  a.dout = tens(dout);
  a.di = di;
  a.lse2 = lse2;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.samples = ws_ptr(workspace, p->off_samples);
  a.H = p->H;
  a.scale = p->scale;
  a.scale_log2 = p->scale * 1.4426950408889634f;
  const bool gf32 = p->desc.grad_dtype == JATTN_F32;
  if (p->dkdv.n_units() > 0 && (stages & JATTN_BWD_DKDV)) {
    a.units = ws_ptr(workspace, p->off_dkdv_u);
    a.worker_off = ws_ptr(workspace, p->off_dkdv_o);
    e = p->D == 128 ? jattn::launch_mx_dkdv_128(a, p->desc.act, gf32, p->dkdv.num_workers, st)
                    : jattn::launch_mx_dkdv_64(a, p->desc.act, gf32, p->dkdv.num_workers, st);
    if (e != hipSuccess) return hip_fail(e, "MXFP8 dK/dV launch");
  }
  if (p->dq.n_units() > 0 && (stages & JATTN_BWD_DQ)) {
    a.units = ws_ptr(workspace, p->off_dq_u);
    a.worker_off = ws_ptr(workspace, p->off_dq_o);
    e = p->D == 128 ? jattn::launch_mx_dq_128(a, p->desc.act, gf32, p->dq.num_workers, st)
                    : jattn::launch_mx_dq_64(a, p->desc.act, gf32, p->dq.num_workers, st);
    if (e != hipSuccess) return hip_fail(e, "MXFP8 dQ launch");
  }
  return ok();
}

int jattn_mx_fwd(const jattn_plan* p, const jattn_mx_tensor* q, const jattn_mx_tensor* k, const jattn_mx_tensor* v,
                 void* o, float* lse, void* workspace, void* stream) {
  if (!p) return fail(JATTN_E_NULL, "null plan");
  if (!p->mx) return fail(JATTN_E_UNSUPPORTED, "not an MXFP8 plan");
  if (p->Tq == 0) return ok();
  if (!q || !k || !v || !o) return fail(JATTN_E_NULL, "null q / k / v / o");
  if (!q->codes || !q->scales || (p->Tk > 0 && (!k->codes || !k->scales || !v->codes_t || !v->scales)))
    return fail(JATTN_E_NULL, "the forward reads q and k codes, v transposed codes and all three scales");
  if (!workspace) return fail(JATTN_E_WORKSPACE, "null workspace");
  if (!aligned(workspace, 256)) return fail(JATTN_E_ALIGN, "workspace must be 256-byte aligned");
  if (!aligned(q->codes, 16) || (p->Tk > 0 && (!aligned(k->codes, 16) || !aligned(v->codes_t, 16))) ||
      !aligned(o, 16) || !aligned(q->scales, 4) || (p->Tk > 0 && (!aligned(k->scales, 4) || !aligned(v->scales, 4))))
    return fail(JATTN_E_ALIGN, "codes and o must be 16-byte aligned, scales 4-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(JATTN_E_ALIGN, "lse must be 4-byte aligned");
  jattn::MxFwdArgs a{};
  auto tens = [](const jattn_mx_tensor* t) {
    return jattn::MxTensor{static_cast<const uint8_t*>(t->codes), static_cast<const uint8_t*>(t->codes_t),
                           static_cast<const uint8_t*>(t->scales)};
  };
  a.q = tens(q);
  a.k = tens(k);
  a.v = tens(v);
  a.o = o;
  a.lse = p->desc.act == JATTN_SOFTMAX ? lse : nullptr;
  a.units = ws_ptr(workspace, p->off_fwd_u);
  a.worker_off = ws_ptr(workspace, p->off_fwd_o);
  a.samples = ws_ptr(workspace, p->off_samples);
  a.H = p->H;
  a.scale = p->scale;
  a.scale_log2 = p->scale * 1.4426950408889634f;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool of32 = p->desc.out_dtype == JATTN_F32;
  const hipError_t e = p->D == 128 ? jattn::launch_mx_fwd_128(a, p->desc.act, of32, p->fwd.num_workers, st)
                                   : jattn::launch_mx_fwd_64(a, p->desc.act, of32, p->fwd.num_workers, st);
  if (e != hipSuccess) return hip_fail(e, "MXFP8 forward launch");
  return ok();
}

namespace {
int l2norm_check(int64_t rows, int32_t D, std::initializer_list<int32_t> dtypes) {
  if (rows < 0) return fail(JATTN_E_SHAPE, "rows must be >= 0");
  if (D != 32 && D != 64 && D != 128) return fail(JATTN_E_SHAPE, "D must be 32, 64 or 128");
  if (rows > (int64_t(1) << 40) / D) return fail(JATTN_E_SHAPE, "too many rows");
  for (int32_t t : dtypes)
    if (t != JATTN_BF16 && t != JATTN_F32) return fail(JATTN_E_UNSUPPORTED, "unknown dtype");
  return JATTN_OK;
}
}  // namespace

int jattn_l2norm_fwd(const void* x, void* y, float* rnorm, int64_t rows, int32_t D, int32_t x_dtype,
                     int32_t y_dtype, void* stream) {
  const int c = l2norm_check(rows, D, {x_dtype, y_dtype});
  if (c != JATTN_OK) return c;
  if (rows == 0) return ok();
  if (!x || !y) return fail(JATTN_E_NULL, "null x/y");
  if (!aligned(x, 16) || !aligned(y, 16) || (rnorm && !aligned(rnorm, 4)))
    return fail(JATTN_E_ALIGN, "x/y must be 16-byte aligned, rnorm 4-byte aligned");
  const hipError_t e = jattn::launch_l2norm_fwd(x, y, rnorm, rows, D, x_dtype == JATTN_F32, y_dtype == JATTN_F32,
                                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "l2norm forward launch");
  return ok();
}

int jattn_l2norm_bwd(const void* x, const void* dy, void* dx, int64_t rows, int32_t D, int32_t x_dtype,
                     int32_t dy_dtype, int32_t dx_dtype, void* stream) {
  const int c = l2norm_check(rows, D, {x_dtype, dy_dtype, dx_dtype});
  if (c != JATTN_OK) return c;
  if (rows == 0) return ok();
  if (!x || !dy || !dx) return fail(JATTN_E_NULL, "null x/dy/dx");
  if (!aligned(x, 16) || !aligned(dy, 16) || !aligned(dx, 16)) return fail(JATTN_E_ALIGN, "x/dy/dx must be 16-byte aligned");
  const hipError_t e = jattn::launch_l2norm_bwd(x, dy, dx, rows, D, x_dtype == JATTN_F32, dy_dtype == JATTN_F32,
                                                dx_dtype == JATTN_F32, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "l2norm backward launch");
  return ok();
}

}  // extern "C"

namespace jattn {

hipError_t launch_fwd(const FwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  if (k.in_f32) {
    if (k.D == 64) return launch_fwd_64_f32_f32(a, k, grid, st);
    return launch_fwd_32_f32_f32(a, k, grid, st);
  }
  if (k.D == 128) return launch_fwd2_128(a, k, grid, st);
  if (k.D == 64) return launch_fwd2_64(a, k, grid, st);
  return launch_fwd2_32(a, k, grid, st);
}

hipError_t launch_dq(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  if (k.in_f32) {
    if (k.D == 64) return launch_dq_64_f32_f32(a, k, grid, st);
    return launch_dq_32_f32_f32(a, k, grid, st);
  }
  if (k.out_f32) {
    if (k.D == 128) return launch_dq2_128_f32(a, k, grid, st);
    if (k.D == 64) return launch_dq2_64_f32(a, k, grid, st);
    return launch_dq2_32_f32(a, k, grid, st);
  }
  if (k.D == 128) return launch_dq2_128_bf16(a, k, grid, st);
  if (k.D == 64) return launch_dq2_64_bf16(a, k, grid, st);
  return launch_dq2_32_bf16(a, k, grid, st);
}

hipError_t launch_dkdv(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  if (k.in_f32) {
    if (k.D == 64) return launch_dkdv_64_f32_f32(a, k, grid, st);
    return launch_dkdv_32_f32_f32(a, k, grid, st);
  }
  // softmax (dense mask or window) with 128-key units at D = 128: two waves
  // per key block (P and dV; dP, dS and dK), two waves per SIMD
  if (k.D == 128 && k.act == JATTN_SOFTMAX && !k.split && k.wkv == 4)
    return k.out_f32 ? launch_dkdv_pair_128_f32(a, k, grid, st) : launch_dkdv_pair_128_bf16(a, k, grid, st);
  if (k.out_f32) {
    if (k.D == 128) return launch_dkdv2_128_f32(a, k, grid, st);
    if (k.D == 64) return launch_dkdv2_64_f32(a, k, grid, st);
    return launch_dkdv2_32_f32(a, k, grid, st);
  }
  if (k.D == 128) return launch_dkdv2_128_bf16(a, k, grid, st);
  if (k.D == 64) return launch_dkdv2_64_bf16(a, k, grid, st);
  return launch_dkdv2_32_bf16(a, k, grid, st);
}

hipError_t launch_di(const DiArgs& a, const KernelSel& k, bool o_f32, hipStream_t st) {
  if (k.in_f32) {
    if (k.D == 64) return launch_di_64_f32(a, o_f32, st);
    return launch_di_32_f32(a, o_f32, st);
  }
  if (k.D == 128) return launch_di_128_bf16(a, o_f32, st);
  if (k.D == 64) return launch_di_64_bf16(a, o_f32, st);
  return launch_di_32_bf16(a, o_f32, st);
}

}  // namespace jattn
