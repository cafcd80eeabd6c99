// Device-side building blocks of the verify-step kernels (gfx950, wave64).
//
// Exponentials.  p(x) = exp((x - xmax) / T) / sum(...) is the temperature
// softmax of [WR] §7.2; any reference R >= max(x * log2(e) / T) gives the
// same p, and an integral R lets partial sums taken against different
// references be merged exactly with ldexp.  Three forms of one exponential
// are used, each where its accuracy is enough (so that a value computed in
// two kernels is bit-identical, a kernel always uses the form its
// consumers use):
//   c      = log2(e) / T rounded to a float; c2 + cl the same as a float
//            just below it plus the (positive) float of the remainder
//            (computed once on the host from the double c64)
//   R      = ceilf(xmax * c)                     (integral float, per row)
//   e(x)   = exp2(fma(x, c, -R))                 (float: the truncated rows'
//            streaming pass, top-p masses)
//   e2(x)  = exp2(fma(x, cl, fma(x, c2, -R)))    (float with the two-part c:
//            the untruncated rows' sums S and their acceptance test)
//   e64(x) = exp2(x * c64 - R)                   (double: the kept sets' sums
//            S64, every draw and every statistic)
// The float forms carry a relative error of a few 1e-7 per term, which is
// harmless to decisions compared against a uniform (acceptance, top-p
// cut) but not to a residual (p - q)+ whose total may be small, nor to
// statistics asked for to 1e-5 relative; those use e64 against S64, the
// double sum of e64 over the kept set.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kWave = 64;
constexpr float kNegInf = -__builtin_inff();
constexpr float kPosInf = __builtin_inff();
constexpr float kLowest = -3.40282346638528859812e+38f;  // -FLT_MAX

// ---- chunk / row flags (internal) ----------------------------------------
constexpr uint32_t CF_NAN = 1u;       // a NaN logit was seen
constexpr uint32_t CF_POSINF = 2u;    // a +Inf logit was seen
constexpr uint32_t CF_OVERFLOW = 4u;  // candidate buffer could not hold the ties

constexpr uint32_t RF_NONFINITE = 1u;  // row unusable (NaN / +Inf / all -Inf)
constexpr uint32_t RF_BIG = 4u;        // kept set not stored as a list: full-row passes

// Per (row, chunk) result of the streaming pass.
struct alignas(16) ChunkOut {
  float xmax;      // max over the chunk (NaN ignored); -inf if none
  int32_t argmax;  // first index (within the row) holding xmax
  float thr;       // every finite chunk element >= thr is in the candidate list
  int32_t ncand;   // candidates written for this chunk
  double s;        // sum over the chunk of exp2(x * c - Rs)
  float Rs;        // integral reference of s; -inf when nothing finite was seen
  uint32_t flags;  // CF_*
};

struct alignas(8) Cand {
  float v;
  int32_t idx;
};

// Per row result of the finalisation (kept set and draft gather).
struct alignas(16) RowInfo {
  double S;        // normaliser of the float exponentials over the kept set
                   // (e2 on untruncated rows, e on truncated ones), reference R
  double S64;      // sum of e64 over the kept set; 0 when not known (untruncated
                   // rows: the passes that need it sum it themselves)
  float R;         // integral reference
  float tau;       // kept set = {x : z(x) >= tau}; kLowest keeps every finite x
  int32_t nkept;   // length of the stored kept list, -1 for RF_BIG rows
  uint32_t flags;  // RF_*
  float ed;        // e2(d) of this row's draft (0 if not kept / bad id / no draft)
  float qd;        // q(d) of this row's draft
  int32_t d;       // draft id; -1 for the bonus row; -2 for an id outside [0, V)
  float zd;        // the draft's logit z(d) (when d >= 0)
};

// A request whose token must be drawn by the full-row sampler.
struct alignas(16) BigJob {
  double S;          // normaliser of the float exponentials (classification only)
  double S64;        // sum of e64 over the kept set, 0 when not known
  float R;
  float tau;
  float u;
  int32_t row;       // target tensor row of the sampled position
  int32_t qrow;      // q row (draft position) when residual, else -1
  int32_t slot;      // output slot (= n_accepted)
  int32_t active;
  int32_t pad;
};

// ---- where a request's rows sit in the caller's arrays -------------------------
// Uniform batches (cu == null): every request has gamma drafts, at draft
// positions [b * gamma, b * gamma + gamma).  Ragged batches (the draft
// length is chosen per request, [WR] §11.2, [MN] §九): request b's
// gamma_b = cu[b+1] - cu[b] drafts are positions [cu[b], cu[b+1]) of packed
// arrays holding n_draft drafts, and gamma bounds every gamma_b.  Either way
// request b's target rows (and resampling uniforms) are rows
// lo + b .. lo + b + gamma_b of the packed target tensor (one more row than
// drafts).  A ragged span that is out of order, out of range or longer than
// gamma is never used (ok = false).
struct Layout {
  const int32_t* cu;  // [B + 1] draft offsets, or null (uniform)
  int32_t n_draft;
  int32_t gamma;
};
struct Span {
  int32_t lo, g;
  bool ok;
};
__device__ __forceinline__ Span span_of(const Layout& L, int b) {
  Span s;
  if (L.cu == nullptr) {
    s.lo = b * L.gamma;
    s.g = L.gamma;
    s.ok = true;
    return s;
  }
  const int32_t lo = L.cu[b], hi = L.cu[b + 1];
  s.ok = 0 <= lo && lo <= hi && hi <= L.n_draft && hi - lo <= L.gamma;
  s.lo = s.ok ? lo : 0;
  s.g = s.ok ? hi - lo : 0;
  return s;
}

// Row r of a row-pass plan: the offset of its logits row, its draft
// position (-1: none, or not gathered here) and whether the row exists.
// Uniform batches: request b = r / rows_per_req, position j; the logits row
// is b * G1 + j and the draft position b * gamma + j (j < gamma).  Ragged
// batches (cu != null, sampling and greedy plans): plan rows are the packed
// target rows themselves, n_live = n_draft + B of them, so the row passes
// need no request index; a grid sized for B * (gamma + 1) rows leaves the
// rest of it idle (those workgroups return before touching memory), and
// the drafts are gathered by the acceptance kernel, which knows each span.
struct RowAt {
  int64_t rowoff, dpos;
  bool live;
};
__device__ __forceinline__ RowAt row_at(const int32_t* cu, int64_t n_live, int rows_per_req, int G1, int gamma,
                                        int64_t V, int64_t r) {
  RowAt o;
  if (cu != nullptr) {
    o.live = r < n_live;
    o.rowoff = r * V;
    o.dpos = -1;
    return o;
  }
  const int64_t b = r / rows_per_req, j = r - b * rows_per_req;
  o.live = true;
  o.rowoff = (b * G1 + j) * V;
  o.dpos = j < gamma ? b * gamma + j : -1;
  return o;
}

// ---- scalar helpers ---------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <bool BF16>
__device__ __forceinline__ void widen(const uint4& w, float* x) {
  if constexpr (BF16) {
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  } else {
    x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
  }
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// The three exponentials against the integral reference R (see the top of
// this file).
__device__ __forceinline__ float e_of(float x, float c, float R) { return ex2(__builtin_fmaf(x, c, -R)); }
// e2 takes the split c2 + cl with c2 below c64 and cl > 0 (not c and the
// signed remainder): then x = -inf gives -inf + -inf and 2^-inf = 0 (with a
// negative low part -inf * cl would be +inf and +inf - inf a NaN).
__device__ __forceinline__ float e2_of(float x, float c2, float cl, float R) {
  return ex2(__builtin_fmaf(x, cl, __builtin_fmaf(x, c2, -R)));
}
// 2^t in double for t <= ~2: 2^n e^g with n = rint(t), g = (t - n) ln 2,
// |g| <= 0.347, and e^g by its Taylor series through g^13 (the first term
// left out is below 1e-17), evaluated by Horner's rule with the
// coefficients as scalar operands (no vector registers held for them).
// Below t = -1100 (-inf included) the result is 0; NaN stays NaN.
__device__ __forceinline__ double exp2_d(double t) {
  if (t < -1100.0) return 0.0;
  const double n = __builtin_rint(t);
  const double g = (t - n) * 0.6931471805599453094;
  double p = 1.0 / 6227020800.0;              // 1/13!
  p = __builtin_fma(p, g, 1.0 / 479001600.0);  // 1/12!
  p = __builtin_fma(p, g, 1.0 / 39916800.0);
  p = __builtin_fma(p, g, 1.0 / 3628800.0);
  p = __builtin_fma(p, g, 1.0 / 362880.0);
  p = __builtin_fma(p, g, 1.0 / 40320.0);
  p = __builtin_fma(p, g, 1.0 / 5040.0);
  p = __builtin_fma(p, g, 1.0 / 720.0);
  p = __builtin_fma(p, g, 1.0 / 120.0);
  p = __builtin_fma(p, g, 1.0 / 24.0);
  p = __builtin_fma(p, g, 1.0 / 6.0);
  p = __builtin_fma(p, g, 0.5);
  p = __builtin_fma(p, g, 1.0);
  p = __builtin_fma(p, g, 1.0);
  const double nc = __builtin_fmax(n, -2000.0);  // keeps the int conversion in range
  return __builtin_ldexp(p, (int)nc);
}
__device__ __forceinline__ double e64_of(float x, double c64, float R) {
  return exp2_d(__builtin_fma((double)x, c64, -(double)R));
}

// A 16-byte load of data that is streamed and read once: the non-temporal
// form, which also streams from HBM faster than a plain load on this part
// (0.85 against 0.79 of peak on a 4 GB read).
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <bool BF16>
__device__ __forceinline__ float load_logit(const void* p, int64_t i) {
  if constexpr (BF16) {
    uint32_t h = reinterpret_cast<const uint16_t*>(p)[i];
    return __uint_as_float(h << 16);
  } else {
    return reinterpret_cast<const float*>(p)[i];
  }
}

// ---- the draft distribution q -----------------------------------------------
// q is either a dense float32 tensor [B * gamma][V] handed over by the caller,
// or the draft's logits [B * gamma][V] processed by the same rules as the
// target's ([WR] §2.3: p and q are both the distributions after the decoding
// rules): q_j(x) = e_j(z(x)) / S_j on the draft row's kept set {z >= tau_j},
// 0 elsewhere, from that row's statistics (S, S64, R, tau) found by the same
// row passes.  A draft row without usable statistics (NaN / +Inf logits, or
// all -Inf) gives q = NaN.
struct QSrc {
  const float* dense;   // dense q, or null
  const void* z;        // draft logits when dense is null; both null: no q (reads give 0)
  const RowInfo* info;  // statistics of the draft rows (with z)
  int64_t V;
  float c, c2, cl;      // log2(e) / T: c for e; c2 + cl for e2 (shared with the target)
  double c64;           // log2(e) / T
  int32_t zbf16;        // the draft logits are bfloat16
};

// One q row.  Values are read "raw" (the dense q, or the draft's logit) and
// turned into q by the accessor the caller's precision asks for.
struct QRow {
  const float* dense;  // start of the dense row, or null
  const void* z;
  int64_t zoff;        // element offset of the row in z
  double invS;         // 1 / S (float exponentials)
  double invS64;       // 1 / S64, 0 when S64 is not known (untruncated draft rows)
  double S64;          // S64 itself (0 when not known)
  double c64;
  float R, tau, c, c2, cl;
  int32_t zbf16;
  int32_t bad;         // unusable draft row: q is NaN

  __device__ __forceinline__ bool logits_src() const { return dense == nullptr && z != nullptr; }

  // q of a draft logit as a float (the acceptance test's q(d)): e64 / S64
  // where S64 is known, else the float exponential that S sums.
  __device__ __forceinline__ float from_logit(float zz) const {
    if (bad) return __builtin_nanf("");
    if (!(zz >= tau)) return 0.0f;
    if (invS64 > 0.0) return (float)(e64_of(zz, c64, R) * invS64);
    return (float)((double)e2_of(zz, c2, cl, R) * invS);
  }
  // q in double from a raw value (needs S64 for draft logits).
  __device__ __forceinline__ double q64(float v) const {
    if (dense) return (double)v;
    if (z == nullptr) return 0.0;
    if (bad) return __builtin_nan("");
    return v >= tau ? e64_of(v, c64, R) * invS64 : 0.0;
  }
  // The same by a true division e64 / S64 (the statistics: a one-token
  // distribution is then exactly 1, as in the plain definition).
  __device__ __forceinline__ double q64_div(float v) const {
    if (dense) return (double)v;
    if (z == nullptr) return 0.0;
    if (bad) return __builtin_nan("");
    return v >= tau ? e64_of(v, c64, R) / S64 : 0.0;
  }
  // The unnormalised double weight of a raw value: q itself for a dense
  // row, e64 of the logit for draft logits (whose normaliser the caller
  // sums itself).
  __device__ __forceinline__ double e64raw(float v) const {
    if (dense) return (double)v;
    if (z == nullptr) return 0.0;
    if (bad) return __builtin_nan("");
    return v >= tau ? e64_of(v, c64, R) : 0.0;
  }
  // An approximation of q from e64raw(v), good to a few 1e-7: enough to
  // tell on which side of p a term lies (the exact sums come from e64raw).
  __device__ __forceinline__ double approx(double e64r) const { return logits_src() ? e64r * invS : e64r; }

  __device__ __forceinline__ float raw_at(int64_t x) const {
    if (dense) return dense[x];
    if (z == nullptr) return 0.0f;
    return zbf16 ? load_logit<true>(z, zoff + x) : load_logit<false>(z, zoff + x);
  }
  __device__ __forceinline__ float at(int64_t x) const {
    if (dense) return dense[x];
    if (z == nullptr) return 0.0f;
    return from_logit(raw_at(x));
  }
  __device__ __forceinline__ double at64(int64_t x) const { return q64(raw_at(x)); }

  // Raw values at x0 .. x0+7 of a whole segment whose 16-byte loads the
  // caller knows to be aligned (dense rows: row * V + x0 a multiple of 4;
  // logits: of 8 for bf16, 4 for fp32).  Straight-line code, so that a
  // caller's unrolled loop keeps several segments' loads in flight.
  __device__ __forceinline__ void raw8_whole(int64_t x0, float* v) const {
    if (dense) {
      const uint4* p = reinterpret_cast<const uint4*>(dense + x0);
      widen<false>(p[0], v);
      widen<false>(p[1], v + 4);
      return;
    }
    const int64_t o = zoff + x0;
    if (zbf16) {
      widen<true>(reinterpret_cast<const uint4*>(z)[o >> 3], v);
    } else {
      const uint4* p = reinterpret_cast<const uint4*>(z) + (o >> 2);
      widen<false>(p[0], v);
      widen<false>(p[1], v + 4);
    }
  }
  // Raw values at x0 .. x0+7 past which (>= V) a dense row reads 0 and draft
  // logits -inf (both: q = 0); 16-byte loads where the segment is whole and
  // aligned.  A row view without q reads 0.
  __device__ __forceinline__ void raw8(int64_t x0, int64_t V, float* v) const {
    const bool full = x0 + 8 <= V;
    if (dense) {
      const float* p = dense + x0;
      if (full && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
        widen<false>(reinterpret_cast<const uint4*>(p)[0], v);
        widen<false>(reinterpret_cast<const uint4*>(p)[1], v + 4);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = (x0 + k < V) ? p[k] : 0.0f;
      }
      return;
    }
    if (z == nullptr) {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = 0.0f;
      return;
    }
    const int64_t o = zoff + x0;
    if (zbf16) {
      if (full && (o & 7) == 0) {
        widen<true>(reinterpret_cast<const uint4*>(z)[o >> 3], v);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = (x0 + k < V) ? load_logit<true>(z, o + k) : kNegInf;
      }
    } else {
      if (full && (o & 3) == 0) {
        const uint4* p = reinterpret_cast<const uint4*>(z) + (o >> 2);
        widen<false>(p[0], v);
        widen<false>(p[1], v + 4);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = (x0 + k < V) ? load_logit<false>(z, o + k) : kNegInf;
      }
    }
  }
};

__device__ __forceinline__ QRow q_row(const QSrc& s, int64_t row) {
  QRow r;
  r.dense = s.dense ? s.dense + row * s.V : nullptr;
  r.z = s.dense ? nullptr : s.z;
  r.zoff = row * s.V;
  r.c = s.c;
  r.c2 = s.c2;
  r.cl = s.cl;
  r.c64 = s.c64;
  r.zbf16 = s.zbf16;
  r.invS = 0.0;
  r.invS64 = 0.0;
  r.S64 = 0.0;
  r.R = 0.0f;
  r.tau = kLowest;
  r.bad = 0;
  if (r.z != nullptr) {
    const RowInfo ri = s.info[row];
    r.bad = (ri.flags & RF_NONFINITE) ? 1 : 0;
    r.invS = 1.0 / ri.S;
    r.invS64 = ri.S64 > 0.0 ? 1.0 / ri.S64 : 0.0;
    r.S64 = ri.S64;
    r.R = ri.R;
    r.tau = ri.tau;
  }
  return r;
}

// A row view that reads 0 everywhere (no q: bonus draws).
__device__ __forceinline__ QRow q_none() {
  QRow r;
  r.dense = nullptr;
  r.z = nullptr;
  r.zoff = 0;
  r.invS = 0.0;
  r.invS64 = 0.0;
  r.S64 = 0.0;
  r.c64 = 0.0;
  r.R = 0.0f;
  r.tau = kLowest;
  r.c = 0.0f;
  r.c2 = 0.0f;
  r.cl = 0.0f;
  r.zbf16 = 0;
  r.bad = 0;
  return r;
}

__device__ __forceinline__ float q_at(const QSrc& s, int64_t row, int64_t x) { return q_row(s, row).at(x); }

// Order-preserving key of a float (-0 folded onto +0, so keys of equal
// values are equal).
__device__ __forceinline__ uint32_t f2key(float f) {
  uint32_t b = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) {
  uint32_t b = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(b);
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Orders LDS traffic of one wave without a workgroup barrier.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- wave reductions / scans over DPP (fixed order: deterministic) --------
// Cross-lane moves use the data-parallel primitives of the VALU (DPP: the
// source lane is picked by a fixed pattern inside the instruction), not the
// LDS crossbar, so one step costs a move and an add instead of an LDS round
// trip.  Patterns used (CDNA encodings): quad_perm within groups of 4 lanes,
// row_shr:n (lane l of a 16-lane row reads lane l - n of that row),
// row_half_mirror and row_mirror (lane l reads 7 - l / 15 - l within its
// half-row / row), row_bcast:15 and row_bcast:31 (the last lane of row r,
// resp. of rows 0-1, is read by the rows the row mask selects), and wave_shr:1
// (lane l reads lane l - 1 of the whole wave).  Lanes whose source lies
// outside the pattern's range, or whose row the mask leaves out, keep `old`.
// Every caller runs these with all 64 lanes active.
enum : int {
  kDppQuadSwap1 = 0xB1,  // quad_perm [1,0,3,2]: lane l reads l ^ 1
  kDppQuadSwap2 = 0x4E,  // quad_perm [2,3,0,1]: lane l reads l ^ 2
  kDppRowShr = 0x110,    // + n: row_shr:n
  kDppRowMirror = 0x140,
  kDppRowHalfMirror = 0x141,
  kDppRowBcast15 = 0x142,
  kDppRowBcast31 = 0x143,
  kDppWaveShr1 = 0x138,
};

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xf, false);
}
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_i32(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xf, false);
}
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f32(float old, float v) {
  return __uint_as_float(dpp_u32<CTRL, ROW_MASK>(__float_as_uint(old), __float_as_uint(v)));
}
// 64-bit values move as two 32-bit halves under the same pattern.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long old, unsigned long long v) {
  const uint32_t lo = dpp_u32<CTRL, ROW_MASK>((uint32_t)old, (uint32_t)v);
  const uint32_t hi = dpp_u32<CTRL, ROW_MASK>((uint32_t)(old >> 32), (uint32_t)(v >> 32));
  return ((unsigned long long)hi << 32) | lo;
}
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp_f64(double old, double v) {
  return __longlong_as_double(
      (long long)dpp_u64<CTRL, ROW_MASK>((unsigned long long)__double_as_longlong(old),
                                         (unsigned long long)__double_as_longlong(v)));
}

// Lane 63's value, uniform over the wave.
__device__ __forceinline__ int wave_last_i(int v) { return __builtin_amdgcn_readlane(v, kWave - 1); }
__device__ __forceinline__ uint32_t wave_last_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}
__device__ __forceinline__ float wave_last_f(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}
__device__ __forceinline__ unsigned long long wave_last_u64(unsigned long long v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, kWave - 1);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), kWave - 1);
  return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ double wave_last_d(double v) {
  return __longlong_as_double((long long)wave_last_u64((unsigned long long)__double_as_longlong(v)));
}

// Lane l - 1's value (lane 0: `first`).
__device__ __forceinline__ double wave_prev_d(double v, double first) { return dpp_f64<kDppWaveShr1>(first, v); }
__device__ __forceinline__ int wave_prev_i(int v, int first) { return dpp_i32<kDppWaveShr1>(first, v); }

// Reduction: quad swaps and the two mirrors leave every lane of a 16-lane
// row with its row's result; the broadcasts fold row 0 into row 1, row 2
// into row 3, then rows 0-1 into rows 2-3, so lane 63 ends with
// (r3 . r2) . (r1 . r0), which is read back to all lanes.  OP(a, b) must be
// commutative (every lane then holds bit-identical row results); ID is its
// identity.
#define SV_WAVE_REDUCE(T, DPP, LAST, OP, ID)            \
  do {                                                   \
    v = OP(v, DPP<kDppQuadSwap1>(ID, v));                \
    v = OP(v, DPP<kDppQuadSwap2>(ID, v));                \
    v = OP(v, DPP<kDppRowHalfMirror>(ID, v));            \
    v = OP(v, DPP<kDppRowMirror>(ID, v));                \
    v = OP(v, DPP<kDppRowBcast15, 0xa>(ID, v));          \
    v = OP(v, DPP<kDppRowBcast31, 0xc>(ID, v));          \
    return LAST(v);                                      \
  } while (0)

__device__ __forceinline__ float op_fmax(float a, float b) { return fmaxf(a, b); }
__device__ __forceinline__ uint32_t op_or(uint32_t a, uint32_t b) { return a | b; }
__device__ __forceinline__ uint32_t op_umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ int op_addi(int a, int b) { return a + b; }
__device__ __forceinline__ double op_addd(double a, double b) { return a + b; }
__device__ __forceinline__ unsigned long long op_addu64(unsigned long long a, unsigned long long b) { return a + b; }

__device__ __forceinline__ float wave_max(float v) { SV_WAVE_REDUCE(float, dpp_f32, wave_last_f, op_fmax, kNegInf); }
__device__ __forceinline__ uint32_t wave_or(uint32_t v) { SV_WAVE_REDUCE(uint32_t, dpp_u32, wave_last_u32, op_or, 0u); }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  SV_WAVE_REDUCE(uint32_t, dpp_u32, wave_last_u32, op_umax, 0u);
}
__device__ __forceinline__ int wave_sum_i(int v) { SV_WAVE_REDUCE(int, dpp_i32, wave_last_i, op_addi, 0); }
__device__ __forceinline__ double wave_sum_d(double v) { SV_WAVE_REDUCE(double, dpp_f64, wave_last_d, op_addd, 0.0); }
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
  SV_WAVE_REDUCE(unsigned long long, dpp_u64, wave_last_u64, op_addu64, 0ull);
}

// Inclusive prefix sum across lanes (lane 0 first): row_shr 1, 2, 4, 8 scan
// each 16-lane row, then the broadcasts carry rows 0, 0-1 and 2 forward.
#define SV_WAVE_SCAN(DPP, ZERO)                     \
  do {                                              \
    v = v + DPP<kDppRowShr + 1>(ZERO, v);           \
    v = v + DPP<kDppRowShr + 2>(ZERO, v);           \
    v = v + DPP<kDppRowShr + 4>(ZERO, v);           \
    v = v + DPP<kDppRowShr + 8>(ZERO, v);           \
    v = v + DPP<kDppRowBcast15, 0xa>(ZERO, v);      \
    v = v + DPP<kDppRowBcast31, 0xc>(ZERO, v);      \
    return v;                                       \
  } while (0)

__device__ __forceinline__ double wave_incl_scan_d(double v) { SV_WAVE_SCAN(dpp_f64, 0.0); }
__device__ __forceinline__ int wave_incl_scan_i(int v) { SV_WAVE_SCAN(dpp_i32, 0); }
__device__ __forceinline__ unsigned long long wave_incl_scan_u64(unsigned long long v) { SV_WAVE_SCAN(dpp_u64, 0ull); }

#undef SV_WAVE_SCAN
#undef SV_WAVE_REDUCE

// (value, index) argmax: larger value wins, equal values keep the lower index.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}
// Argmax over the wave with the same pattern as the reductions (the merge
// is commutative on (value, index) pairs of distinct indices).
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#define SV_ARGMAX_STEP(CTRL, RM)                                                   \
  {                                                                                \
    const float v2 = dpp_f32<CTRL, RM>(kNegInf, v);                                \
    const int i2 = dpp_i32<CTRL, RM>(0x7fffffff, i);                               \
    argmax_merge(v, i, v2, i2);                                                    \
  }
  SV_ARGMAX_STEP(kDppQuadSwap1, 0xf)
  SV_ARGMAX_STEP(kDppQuadSwap2, 0xf)
  SV_ARGMAX_STEP(kDppRowHalfMirror, 0xf)
  SV_ARGMAX_STEP(kDppRowMirror, 0xf)
  SV_ARGMAX_STEP(kDppRowBcast15, 0xa)
  SV_ARGMAX_STEP(kDppRowBcast31, 0xc)
#undef SV_ARGMAX_STEP
  v = wave_last_f(v);
  i = wave_last_i(i);
}

// Exact merge of (s, R) pairs: s * 2^R summed onto the larger reference.
__device__ __forceinline__ void sr_merge(double& s, float& R, double s2, float R2) {
  if (R2 == kNegInf) return;
  if (R == kNegInf) {
    s = s2;
    R = R2;
    return;
  }
  if (R2 > R) {
    s = ldexp(s, (int)(R - R2)) + s2;
    R = R2;
  } else {
    s = s + ldexp(s2, (int)(R2 - R));
  }
}

// Find the radix digit holding the element of rank `need` (1-based, counted
// from the largest) in a 256-bin histogram; executed by one whole wave.
// Returns the digit; `need` becomes the rank inside that digit's bin.
__device__ __forceinline__ int wave_find_digit(const uint32_t* hist, int& need) {
  const int l = lane_id();
  // lane l holds bins 255-4l .. 252-4l (descending)
  uint32_t c0 = hist[255 - 4 * l], c1 = hist[254 - 4 * l], c2 = hist[253 - 4 * l], c3 = hist[252 - 4 * l];
  int lsum = (int)(c0 + c1 + c2 + c3);
  int incl = wave_incl_scan_i(lsum);
  int excl = incl - lsum;
  uint64_t hit = ballot(incl >= need);
  int src = hit ? (int)__builtin_ctzll(hit) : 63;
  int digit = 0, newneed = need;
  if (l == src) {
    int run = excl;
    int cs[4] = {(int)c0, (int)c1, (int)c2, (int)c3};
    int k = 0;
    for (; k < 3; ++k) {
      if (run + cs[k] >= need) break;
      run += cs[k];
    }
    digit = 255 - 4 * l - k;
    newneed = need - run;
  }
  digit = __shfl(digit, src, kWave);
  need = __shfl(newneed, src, kWave);
  return digit;
}

}  // namespace sv
