// K3 / K4 -- the per-request verification and the draws; greedy; statistics.
//
// K3 (one wave per request): acceptance of the gamma drafts left to right,
// accept_j <=> u_accept[j] * q_j(d_j) * S_j < e_j(d_j), i.e. u < p/q in
// exact arithmetic ([WR] §4.1, [BS] §四 rule (1)), evaluated for all j at
// once; the first rejection is the lowest clear bit of a 64-bit ballot
// ([WR] §6: verification is left to right and stops at the first rejection).
// Then the replacement from the residual (p - q)_+ ([WR] §5) or the bonus
// token from p_gamma ([WR] §6): when the kept set of that row is a short
// list the wave draws it at once (inverse CDF, fp64 wave scans); otherwise
// it leaves a BigJob for a full-row draw: by the request's own workgroup on
// truncated rows, else by K4, which sums the weights of a whole row in
// chunks (one launch) and locates the token from the chunk totals (a second
// launch).
#pragma once

#include "sv_device.h"
#include "sv_rowfinal.h"

namespace sv {

// Plan rows: request b's rows are lo + b .. lo + b + gamma_b (lo = its first
// draft position), which is b * (gamma + 1) + j for uniform batches.
struct AcceptArgs {
  RowInfo* info;        // per plan row
  const float2* gath;   // draft gather of the row pass (untruncated rows) or null
  const ChunkOut* cout; // chunk results, read when rows are untruncated (no K2)
  int32_t nchunks;
  const void* logits;
  float c;
  float c2, cl;         // two-part log2(e) / T (untruncated rows' e2)
  double c64;           // log2(e) / T (e64)
  const Cand* kept;     // [rows][kmax]
  int32_t kmax;
  QSrc q;
  const int32_t* ids;
  const float* ua;
  const float* ur;
  int32_t B;
  int32_t gamma;        // (maximum) drafts per request
  int64_t V;
  int32_t* out_tokens;  // [B, gamma + 1]
  int32_t* out_nacc;
  uint32_t* out_flags;  // may be null
  BigJob* jobs;
  const int32_t* cu;    // ragged draft offsets [B + 1], or null (Layout)
  int32_t n_draft;
  int32_t eos;          // end-of-sequence id, < 0: none
  double beta;          // lenience: the draft is compared as beta * q (1: lossless)
};

// Draw from the kept list of one row, stored in token-id order as (logit,
// id) (called by a whole wave).
// residual: weights (p - qs q)_+ on the list (qs = beta), with p = e64 / S64
// and q in double; otherwise p.
// The list is walked 64 entries at a time in id order (prefix sums by wave
// scans, carried between steps); the loads of kDrawBlk steps (list entries,
// then q at their ids) are issued together before their scans.  A list of
// at most kDrawBlk * 64 entries is read once: the total and the search take
// the same registers.  has_pre: the caller already loaded entry `lane`
// (pre) of a list of at most 64 entries.
constexpr int kDrawBlk = 4;
struct DrawBlk {
  Cand e[kDrawBlk];   // entries i0 + 64 k + lane (idx = -1 past the end)
  float qv[kDrawBlk]; // q's raw values at their ids (residual draws)
};

__device__ __forceinline__ void draw_load(const Cand* L, int n, int i0, bool res, const QRow& qr, DrawBlk& d) {
  const int lane = lane_id();
#pragma unroll
  for (int k = 0; k < kDrawBlk; ++k) {
    const int i = i0 + k * kWave + lane;
    d.e[k].v = 0.0f;
    d.e[k].idx = -1;
    if (i < n) d.e[k] = L[i];
  }
#pragma unroll
  for (int k = 0; k < kDrawBlk; ++k) d.qv[k] = (res && d.e[k].idx >= 0) ? qr.raw_at(d.e[k].idx) : 0.0f;
}

__device__ __forceinline__ void draw_weights(const DrawBlk& d, bool res, double invS, float R, double c64,
                                             const QRow& qr, double qs, double (&w)[kDrawBlk]) {
#pragma unroll
  for (int k = 0; k < kDrawBlk; ++k) {
    if (d.e[k].idx < 0) {
      w[k] = 0.0;
    } else {
      const double p = e64_of(d.e[k].v, c64, R) * invS;
      if (!res) {
        w[k] = p;
      } else {
        const double dd = p - qs * qr.q64(d.qv[k]);
        w[k] = dd > 0.0 ? dd : 0.0;
      }
    }
  }
}

__device__ __forceinline__ int draw_from_list(const Cand* L, int n, double S64, float R, double c64, const QRow& qr,
                              bool& residual, float u, uint32_t& fl, double qs, bool has_pre = false,
                              Cand pre = Cand{}) {
  const int lane = lane_id();
  const double invS = 1.0 / S64;
  // sum of one block's weights, carried (the scans of the search below)
  auto blk_total = [&](int i0, const double (&w)[kDrawBlk], double carry) -> double {
#pragma unroll
    for (int k = 0; k < kDrawBlk; ++k) {
      if (i0 + k * kWave >= n) break;
      const double incl = wave_incl_scan_d(w[k]);
      carry = carry + wave_last_d(incl);
    }
    return carry;
  };
  // search of one block from `carry`: the token at the crossing of t, else
  // -1 (lastpos: the last positive entry so far)
  auto blk_search = [&](int i0, const double (&w)[kDrawBlk], const DrawBlk& d, double t, double& carry,
                        int& lastpos) -> int {
#pragma unroll
    for (int k = 0; k < kDrawBlk; ++k) {
      const int j0 = i0 + k * kWave;
      if (j0 >= n) break;
      const int i = j0 + lane;
      const double incl = wave_incl_scan_d(w[k]);
      const double C = carry + incl;
      const uint64_t hit = ballot(i < n && C > t);
      if (hit) return __shfl(d.e[k].idx, (int)__builtin_ctzll(hit), kWave);
      const uint64_t pos = ballot(i < n && w[k] > 0.0);
      if (pos) lastpos = __shfl(d.e[k].idx, 63 - (int)__builtin_clzll(pos), kWave);
      carry = carry + wave_last_d(incl);
    }
    return -1;
  };
  if (n <= kDrawBlk * kWave) {
    DrawBlk d;
    if (has_pre && n <= kWave) {
      d.e[0].v = 0.0f;
      d.e[0].idx = -1;
      if (lane < n) d.e[0] = pre;
#pragma unroll
      for (int k = 1; k < kDrawBlk; ++k) {
        d.e[k].v = 0.0f;
        d.e[k].idx = -1;
      }
#pragma unroll
      for (int k = 0; k < kDrawBlk; ++k) d.qv[k] = (residual && d.e[k].idx >= 0) ? qr.raw_at(d.e[k].idx) : 0.0f;
    } else {
      draw_load(L, n, 0, residual, qr, d);
    }
    double w[kDrawBlk];
    draw_weights(d, residual, invS, R, c64, qr, qs, w);
    double W = blk_total(0, w, 0.0);
    if (residual && !(W > 0.0)) {
      fl |= 4u;  // SV_ROW_Z_DEGENERATE
      residual = false;
      draw_weights(d, false, invS, R, c64, qr, qs, w);
      W = blk_total(0, w, 0.0);
    }
    const double t = (double)u * W;
    double carry = 0.0;
    int lastpos = -1;
    const int token = blk_search(0, w, d, t, carry, lastpos);
    return token >= 0 ? token : lastpos;
  }
  auto total = [&](bool res) -> double {
    double carry = 0.0;
    for (int i0 = 0; i0 < n; i0 += kDrawBlk * kWave) {
      DrawBlk d;
      draw_load(L, n, i0, res, qr, d);
      double w[kDrawBlk];
      draw_weights(d, res, invS, R, c64, qr, qs, w);
      carry = blk_total(i0, w, carry);
    }
    return carry;
  };
  double W = total(residual);
  if (residual && !(W > 0.0)) {
    fl |= 4u;  // SV_ROW_Z_DEGENERATE
    residual = false;
    W = total(false);
  }
  const double t = (double)u * W;
  double carry = 0.0;
  int token = -1, lastpos = -1;
  for (int i0 = 0; i0 < n && token < 0; i0 += kDrawBlk * kWave) {
    DrawBlk d;
    draw_load(L, n, i0, residual, qr, d);
    double w[kDrawBlk];
    draw_weights(d, residual, invS, R, c64, qr, qs, w);
    token = blk_search(i0, w, d, t, carry, lastpos);
  }
  return token >= 0 ? token : lastpos;
}

// Logits (and q's raw values when residual) of tokens x .. x+7 of a row
// (-inf / q = 0 past V).
template <bool BF16>
__device__ __forceinline__ void full_row_seg(const void* logits, const QRow& qr, int64_t rowoff, int64_t V, bool vec,
                                             int64_t x, bool res, float* z, float* qv) {
  if (x >= V) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      z[k] = kNegInf;
      qv[k] = 0.0f;
    }
    return;
  }
  if (vec && x + 8 <= V) {
    if constexpr (BF16) {
      widen<true>(reinterpret_cast<const uint4*>(logits)[(rowoff + x) >> 3], z);
    } else {
      const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(logits) + rowoff + x);
      widen<false>(p[0], z);
      widen<false>(p[1], z + 4);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) z[k] = (x + k < V) ? load_logit<BF16>(logits, rowoff + x + k) : kNegInf;
  }
  if (res) qr.raw8(x, V, qv);
}

// Weight of one token of a row whose S64 is known: e64(z) on the kept set
// {z >= tau}, or the residual (e64 / S64 - qs q)_+ there (q from its raw
// value qraw, in double).
__device__ __forceinline__ double full_row_weight(float z, float qraw, bool res, const QRow& qr, double c64, float R,
                                                  float tau, double invS64, double qs) {
  if (!(z >= tau)) return 0.0;
  const double e = e64_of(z, c64, R);
  if (!res) return e;
  const double d = e * invS64 - qs * qr.q64(qraw);
  return d > 0.0 ? d : 0.0;
}

// Block-wide "first token whose running weight exceeds t, else the last
// token of positive weight" when thread segments are in token order: the
// first hit lives in the lowest wave and lane holding one, the last positive
// token in the highest.  Ballots and one LDS slot per wave, no atomics.
template <int NW>
__device__ int block_first_or_last(int found, int lp, int* s_f, int* s_l) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint64_t hm = ballot(found != 0x7fffffff);
  const int ff = hm ? __shfl(found, (int)__builtin_ctzll(hm), kWave) : 0x7fffffff;
  const uint64_t lm = ballot(lp >= 0);
  const int ll = lm ? __shfl(lp, 63 - (int)__builtin_clzll(lm), kWave) : -1;
  if (lane == 0) {
    s_f[wid] = ff;
    s_l[wid] = ll;
  }
  __syncthreads();
  int tok = -1;
  for (int k = 0; k < NW; ++k)
    if (s_f[k] != 0x7fffffff) {
      tok = s_f[k];
      break;
    }
  if (tok < 0)
    for (int k = NW - 1; k >= 0; --k)
      if (s_l[k] >= 0) {
        tok = s_l[k];
        break;
      }
  return tok;
}

// Shuffle a RowInfo from lane `src`.
__device__ __forceinline__ RowInfo shfl_info(const RowInfo& r, int src) {
  RowInfo o;
  o.S = __shfl(r.S, src, kWave);
  o.S64 = __shfl(r.S64, src, kWave);
  o.R = __shfl(r.R, src, kWave);
  o.tau = __shfl(r.tau, src, kWave);
  o.nkept = __shfl(r.nkept, src, kWave);
  o.flags = __shfl(r.flags, src, kWave);
  o.ed = __shfl(r.ed, src, kWave);
  o.qd = __shfl(r.qd, src, kWave);
  o.d = __shfl(r.d, src, kWave);
  o.zd = __shfl(r.zd, src, kWave);
  return o;
}

// Acceptance test of one draft ([WR] §4.1: accept iff u < p(d) / q(d); here
// u < p(d) / (beta q(d)) with the lenience factor beta, 1 when lossless),
// without a division.  Rows with a known S64 (truncated rows) compare
// e64(d) with u beta q(d) S64 in double; untruncated rows compare e2(d)
// with u beta q(d) S, both from the float exponentials of the row pass
// (a relative error of a few 1e-7 on p(d) / q(d)).  q(d) = 0 accepts iff
// p(d) > 0.
__device__ __forceinline__ bool accept_test(const RowInfo& ri, float ua, double beta, double c64) {
  if (ri.d < 0) return false;
  if (ri.qd == 0.0f) return ri.zd >= ri.tau && e64_of(ri.zd, c64, ri.R) > 0.0;
  if (ri.S64 > 0.0) {
    const double e = ri.zd >= ri.tau ? e64_of(ri.zd, c64, ri.R) : 0.0;
    return (double)ua * (beta * (double)ri.qd) * ri.S64 < e;
  }
  return (double)ua * (beta * (double)ri.qd) * ri.S < (double)ri.ed;
}

// Acceptance decision of one request (whole wave): the first rejection,
// cut at an accepted end-of-sequence draft ([WR] §14.3: nothing is
// committed after an EOS; that draft becomes the last emitted token and no
// token is drawn).
struct Decision {
  int nacc;
  uint32_t fl;
  bool bad;        // emit nothing; badfl says why
  uint32_t badfl;  // SV_ROW_NONFINITE or SV_ROW_BAD_SPAN
  bool eos_cut;
  int lo, G;       // the request's first draft position and gamma_b
  RowInfo rs;      // info of row n_accepted (the row the token is drawn from)
};

// Entry `lane` of the draw row's kept list and that row's resample uniform,
// loaded before the decision was known (see accept_trunc_kernel).
struct ListPick {
  Cand e;
  float u;
};

// Emit the outputs of one request once its decision is known (whole wave).
template <bool BF16>
__device__ __forceinline__ void finish_request(const AcceptArgs& a, int b, const Decision& dc, int32_t* out,
                               bool has_pk = false, ListPick pk = ListPick{}) {
  const int lane = lane_id();
  const int nacc = dc.nacc, G = dc.G, P1 = a.gamma + 1;
  const int64_t lo = dc.lo;
  uint32_t fl = dc.fl;
  const int nids = nacc + (dc.eos_cut ? 1 : 0);  // slots holding draft ids
  for (int jj = lane; jj < P1; jj += kWave)
    if (dc.eos_cut || jj != nacc) out[jj] = jj < nids ? a.ids[lo + jj] : -1;
  if (dc.eos_cut) {
    if (lane == 0) {
      a.out_nacc[b] = nacc;
      if (a.out_flags) a.out_flags[b] = fl;
      a.jobs[b].active = 0;
    }
    return;
  }
  bool residual = nacc < G;
  const float u = has_pk ? pk.u : a.ur[lo + b + nacc];
  const int64_t trow = lo + b + nacc;  // plan row of the draw (= its logits row)
  const int64_t qrow = residual ? lo + nacc : -1;
  const QRow qr = residual ? q_row(a.q, qrow) : q_none();
  const RowInfo& rs = dc.rs;
  if (rs.flags & RF_BIG) {
    if (lane == 0) {
      BigJob jb;
      jb.S = rs.S;
      jb.S64 = rs.S64;
      jb.R = rs.R;
      jb.tau = rs.tau;
      jb.u = u;
      jb.row = (int32_t)trow;
      jb.qrow = (int32_t)qrow;
      jb.slot = nacc;
      jb.active = 1;
      jb.pad = 0;
      a.jobs[b] = jb;
      out[nacc] = -1;  // written by the full-row sampler
      a.out_nacc[b] = nacc;
      if (a.out_flags) a.out_flags[b] = fl;
    }
    return;
  }
  int token = draw_from_list(a.kept + trow * a.kmax, rs.nkept, rs.S64, rs.R, a.c64, qr, residual, u, fl, a.beta,
                             has_pk, pk.e);
  if (lane == 0) {
    if (a.eos >= 0 && token == a.eos) fl |= 16u;  // SV_ROW_EOS
    out[nacc] = token;
    a.out_nacc[b] = nacc;
    if (a.out_flags) a.out_flags[b] = fl;
    a.jobs[b].active = 0;
  }
}

// A request that emits nothing: fl = SV_ROW_NONFINITE or SV_ROW_BAD_SPAN.
__device__ void empty_request(const AcceptArgs& a, int b, int32_t* out, uint32_t fl) {
  const int lane = lane_id();
  for (int jj = lane; jj < a.gamma + 1; jj += kWave) out[jj] = -1;
  if (lane == 0) {
    a.out_nacc[b] = 0;
    if (a.out_flags) a.out_flags[b] = fl;
    a.jobs[b].active = 0;
  }
}

// Acceptance decision of one request with gamma + 1 <= 64 (whole wave, one
// lane per position, all in registers).
template <bool BF16, bool FROM_CHUNKS>
__device__ Decision decide_short(const AcceptArgs& a, int b) {
  const int lane = lane_id();
  const Span sp = span_of(Layout{a.cu, a.n_draft, a.gamma}, b);
  const int G = sp.g;
  RowInfo ri;
  ri.flags = 0;
  ri.d = -1;
  ri.qd = 0.0f;
  ri.ed = 0.0f;
  ri.S = 1.0;
  ri.S64 = 0.0;
  ri.R = 0.0f;
  ri.tau = kLowest;
  ri.nkept = -1;
  ri.zd = 0.0f;
  Decision dc;
  dc.lo = sp.lo;
  dc.G = G;
  dc.eos_cut = false;
  dc.fl = 0;
  dc.nacc = 0;
  if (!sp.ok) {
    dc.bad = true;
    dc.badfl = 32u;  // SV_ROW_BAD_SPAN
    dc.rs = ri;
    return dc;
  }
  float ua = 0.0f;
  if (lane < G) ua = a.ua[(int64_t)sp.lo + lane];
  if (lane <= G) {
    const int64_t prow = (int64_t)sp.lo + b + lane;
    const int64_t dpos = lane < G ? (int64_t)sp.lo + lane : -1;
    if constexpr (FROM_CHUNKS) {
      // ragged rows were not gathered by the row pass: gather here
      ri = untrunc_row_info<BF16>(a.cout + prow * a.nchunks, a.nchunks, a.c, a.c2, a.cl, a.logits, a.q, a.ids, a.V, dpos,
                                  prow * a.V, a.cu != nullptr ? nullptr : a.gath, prow);
    } else {
      ri = a.info[prow];
      if (a.cu != nullptr && !(ri.flags & RF_NONFINITE))
        gather_draft_at<BF16>(a.logits, a.q, a.ids, a.V, a.kept != nullptr ? a.c : a.c2, a.kept != nullptr ? 0.0f : a.cl,
                              dpos, prow * a.V, ri);
    }
  }
  bool bad = (lane <= G) && ((ri.flags & RF_NONFINITE) ||
                              (lane < G && ri.d >= 0 && !(ri.qd >= 0.0f && ri.qd < kPosInf)));
  dc.bad = ballot(bad) != 0;
  dc.badfl = 8u;  // SV_ROW_NONFINITE
  bool acc = true;
  if (lane < G) acc = accept_test(ri, ua, a.beta, a.c64);
  uint64_t rej = ballot(!acc);
  dc.nacc = rej ? (int)__builtin_ctzll(rej) : G;
  if (a.eos >= 0) {
    const uint64_t em = ballot(lane < dc.nacc && ri.d == a.eos);
    if (em) {
      dc.nacc = (int)__builtin_ctzll(em);
      dc.eos_cut = true;
      dc.fl |= 16u;  // SV_ROW_EOS
    }
  }
  if (ballot(lane < G && lane <= dc.nacc && ri.d >= 0 && ri.qd == 0.0f) != 0) dc.fl |= 2u;  // SV_ROW_Q_ZERO
  dc.rs = shfl_info(ri, dc.nacc);
  if (!dc.eos_cut && dc.nacc < G && dc.rs.d == -2) dc.fl |= 1u;  // SV_ROW_BAD_ID
  return dc;
}

// One request's acceptance and draw with gamma + 1 > 64, by one wave: rows
// go through the workspace copy of the row infos (a row whose kept set is
// not a list leaves a BigJob for a full-row draw).
template <bool BF16, bool FROM_CHUNKS>
__device__ __forceinline__ void accept_long(const AcceptArgs& a, int b) {
  const int lane = lane_id();
  const int P1 = a.gamma + 1;
  int32_t* out = a.out_tokens + (int64_t)b * P1;
  const Span sp = span_of(Layout{a.cu, a.n_draft, a.gamma}, b);
  if (!sp.ok) {
    empty_request(a, b, out, 32u);  // SV_ROW_BAD_SPAN
    return;
  }
  const int G = sp.g;
  const int64_t lo = sp.lo;
  RowInfo* inf = a.info + lo + b;
  if constexpr (FROM_CHUNKS) {
    for (int jj = lane; jj <= G; jj += kWave) {
      const int64_t prow = lo + b + jj;
      inf[jj] = untrunc_row_info<BF16>(a.cout + prow * a.nchunks, a.nchunks, a.c, a.c2, a.cl, a.logits, a.q, a.ids, a.V,
                                       jj < G ? lo + jj : -1, prow * a.V);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    wave_sync();
  } else if (a.cu != nullptr) {
    // ragged rows were not gathered by the row finisher: gather here
    for (int jj = lane; jj <= G; jj += kWave) {
      RowInfo ri = inf[jj];
      if (!(ri.flags & RF_NONFINITE))
        gather_draft_at<BF16>(a.logits, a.q, a.ids, a.V, a.kept != nullptr ? a.c : a.c2, a.kept != nullptr ? 0.0f : a.cl,
                              jj < G ? lo + jj : -1,
                              (lo + b + jj) * a.V, ri);
      inf[jj] = ri;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    wave_sync();
  }
  bool bad = false;
  for (int jj = lane; jj <= G; jj += kWave) {
    RowInfo ri = inf[jj];
    if (ri.flags & RF_NONFINITE) bad = true;
    if (jj < G && ri.d >= 0 && !(ri.qd >= 0.0f && ri.qd < kPosInf)) bad = true;
  }
  if (ballot(bad) != 0) {
    empty_request(a, b, out, 8u);  // SV_ROW_NONFINITE
    return;
  }
  int nacc = G;
  for (int j0 = 0; j0 < G; j0 += kWave) {
    const int jj = j0 + lane;
    bool acc = true;
    if (jj < G) acc = accept_test(inf[jj], a.ua[lo + jj], a.beta, a.c64);
    uint64_t rej = ballot(!acc);
    if (rej) {
      nacc = j0 + (int)__builtin_ctzll(rej);
      break;
    }
  }
  Decision dc;
  dc.fl = 0;
  dc.eos_cut = false;
  if (a.eos >= 0) {
    for (int j0 = 0; j0 < nacc; j0 += kWave) {
      const int jj = j0 + lane;
      const uint64_t em = ballot(jj < nacc && inf[jj].d == a.eos);
      if (em) {
        nacc = j0 + (int)__builtin_ctzll(em);
        dc.eos_cut = true;
        dc.fl |= 16u;  // SV_ROW_EOS
        break;
      }
    }
  }
  bool qz = false;
  for (int jj = lane; jj < min(nacc + 1, G); jj += kWave) {
    RowInfo ri = inf[jj];
    if (ri.d >= 0 && ri.qd == 0.0f) qz = true;
  }
  if (ballot(qz) != 0) dc.fl |= 2u;  // SV_ROW_Q_ZERO
  dc.rs = inf[nacc];
  if (!dc.eos_cut && nacc < G && dc.rs.d == -2) dc.fl |= 1u;  // SV_ROW_BAD_ID
  dc.nacc = nacc;
  dc.bad = false;
  dc.badfl = 0;
  dc.lo = sp.lo;
  dc.G = G;
  finish_request<BF16>(a, b, dc, out);
}

// Untruncated rows with gamma + 1 > 64: four requests per workgroup, one per
// wave (the full-row draws are BigJobs for the chunked sampler).
template <bool BF16>
__global__ void __launch_bounds__(256) accept_kernel(AcceptArgs a) {
  const int b = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (b >= a.B) return;
  accept_long<BF16, true>(a, b);
}

// Truncated rows: one request per workgroup.  Wave 0 takes the decision and
// draws from a kept list; a row whose kept set is too large for a list (a
// wide nucleus) is drawn by the whole workgroup, one quarter of the row per
// wave: each wave totals its quarter, and the wave whose quarter holds the
// crossing of t = u * W finds the token (sums in a fixed order).
//
// Requests of at most kPfRows rows: while wave 0 reads the row infos and
// takes the decision, waves 1-3 copy the first 64 entries of every row's
// kept list and every row's resample uniform into LDS, so that once the
// draw row is known a list of up to 64 entries costs no further round trip
// but q at its ids (entries past the row's nkept are never used).  Waves 1-3
// leave as soon as the decision shows that the draw row has a list.
constexpr int kPfRows = 8;
template <bool BF16>
__global__ void __launch_bounds__(256, 4) accept_trunc_kernel(AcceptArgs a) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int b = blockIdx.x;
  __shared__ double s_tot[4];
  __shared__ long long s_tok;
  __shared__ Cand s_pre[kPfRows * kWave];
  __shared__ float s_ur[kPfRows];
  __shared__ int s_big;
  if (a.gamma + 1 <= kWave) {
    const bool pf = a.gamma + 1 <= kPfRows;
    Decision dc;
    if (wid == 0) {
      dc = decide_short<BF16, false>(a, b);
      // the draw row's kept set is not a list: the four waves draw it below
      if (lane == 0) s_big = (!dc.bad && !dc.eos_cut && (dc.rs.flags & RF_BIG)) ? 1 : 0;
    } else if (pf) {
      const Span sp = span_of(Layout{a.cu, a.n_draft, a.gamma}, b);
      if (sp.ok) {
        const int t = (int)threadIdx.x - kWave;
        for (int i = t; i < (sp.g + 1) * kWave; i += 3 * kWave)
          s_pre[i] = a.kept[((int64_t)sp.lo + b + (i >> 6)) * a.kmax + (i & 63)];
        if (t <= sp.g) s_ur[t] = a.ur[(int64_t)sp.lo + b + t];
      }
    }
    __syncthreads();
    const bool big = s_big != 0;
    if (wid != 0 && !big) return;  // nothing left for waves 1-3
    if (wid == 0) {
      int32_t* out = a.out_tokens + (int64_t)b * (a.gamma + 1);
      if (dc.bad) {
        empty_request(a, b, out, dc.badfl);
      } else {
        ListPick pk;
        pk.e.v = 0.0f;
        pk.e.idx = -1;
        pk.u = 0.0f;
        if (pf) {
          pk.e = s_pre[dc.nacc * kWave + lane];
          pk.u = s_ur[dc.nacc];
        }
        finish_request<BF16>(a, b, dc, out, pf, pk);
      }
    }
    if (!big) return;
    __syncthreads();  // wave 0 has stored the request's BigJob
  } else {
    if (wid == 0) accept_long<BF16, false>(a, b);
    __syncthreads();
  }
  const BigJob jb = a.jobs[b];
  if (!jb.active) return;
  const int64_t V = a.V;
  const int64_t rowoff = (int64_t)jb.row * V;
  const bool vec = (rowoff % (BF16 ? 8 : 4)) == 0;
  bool residual = jb.qrow >= 0;
  const QRow qr = residual ? q_row(a.q, jb.qrow) : q_none();
  constexpr int64_t kStep = 8 * kWave;
  const int64_t Lq = (V + 4 * kStep - 1) / (4 * kStep) * kStep;  // a quarter, whole steps
  const int64_t q0 = min((int64_t)wid * Lq, V), q1 = min(q0 + Lq, V);
  const double invS64 = 1.0 / jb.S64;  // truncated rows always carry S64
  // this wave's quarter: its total (t < 0), or the search from `carry`
  struct QOut {
    double carry;
    int64_t token, lastpos;
  };
  auto quarter = [&](bool res, double t, double carry) -> QOut {
    int64_t token = -1, lastpos = -1;
    for (int64_t x0 = q0; x0 < q1; x0 += kStep) {
      const int64_t x = x0 + (int64_t)lane * 8;
      const bool in = x < q1;
      float z[8], qv[8];
      full_row_seg<BF16>(a.logits, qr, rowoff, in ? V : 0, vec, x, res, z, qv);
      double seg = 0.0;
      int lastk = -1;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const double wk = full_row_weight(z[k], qv[k], res, qr, a.c64, jb.R, jb.tau, invS64, a.beta);
        seg += wk;
        if (wk > 0.0) lastk = k;
      }
      const double incl = wave_incl_scan_d(seg);
      if (t >= 0.0) {
        const double C = carry + incl;
        const double ex = wave_prev_d(C, carry);
        const uint64_t hit = ballot(in && C > t);
        if (hit) {
          const int src = (int)__builtin_ctzll(hit);
          int64_t found = -1;
          if (lane == src) {
            double run = ex;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              run = run + full_row_weight(z[k], qv[k], res, qr, a.c64, jb.R, jb.tau, invS64, a.beta);
              if (found < 0 && run > t) found = x + k;
            }
            if (found < 0) found = x + lastk;  // rounding: the lane's last positive token
          }
          token = __shfl(found, src, kWave);
          return QOut{carry, token, lastpos};
        }
        const uint64_t pos = ballot(in && lastk >= 0);
        if (pos) lastpos = __shfl(x + lastk, 63 - (int)__builtin_clzll(pos), kWave);
      }
      carry = carry + wave_last_d(incl);
    }
    return QOut{carry, token, lastpos};
  };
  uint32_t extra = 0;
  double tq = quarter(residual, -1.0, 0.0).carry;
  if (lane == 0) s_tot[wid] = tq;
  __syncthreads();
  double W = ((s_tot[0] + s_tot[1]) + s_tot[2]) + s_tot[3];
  if (residual && !(W > 0.0)) {
    extra |= 4u;  // SV_ROW_Z_DEGENERATE: draw from p instead
    residual = false;
    __syncthreads();
    tq = quarter(false, -1.0, 0.0).carry;
    if (lane == 0) s_tot[wid] = tq;
    __syncthreads();
    W = ((s_tot[0] + s_tot[1]) + s_tot[2]) + s_tot[3];
  }
  const double t = (double)jb.u * W;
  // the quarter holding the crossing (running totals in the order of W),
  // else the last quarter of positive weight (whose last positive token is
  // the draw)
  int kq = -1, lastq = -1;
  double before = 0.0, cum = 0.0, before_last = 0.0;
  for (int k = 0; k < 4; ++k) {
    if (s_tot[k] > 0.0) {
      lastq = k;
      before_last = cum;
    }
    if (kq < 0 && cum + s_tot[k] > t) {
      kq = k;
      before = cum;
    }
    cum = cum + s_tot[k];
  }
  if (threadIdx.x == 0) s_tok = -1;
  __syncthreads();
  if (kq >= 0 && wid == kq) {
    const QOut r = quarter(residual, t, before);
    if (lane == 0) s_tok = r.token >= 0 ? r.token : r.lastpos;
  } else if (kq < 0 && lastq >= 0 && wid == lastq) {
    const QOut r = quarter(residual, 1.0 / 0.0, before_last);  // no crossing: the last positive token
    if (lane == 0) s_tok = r.lastpos;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int token = (int)s_tok;
    a.out_tokens[(int64_t)b * (a.gamma + 1) + jb.slot] = token;
    if (a.eos >= 0 && token == a.eos) extra |= 16u;  // SV_ROW_EOS
    if (extra && a.out_flags) a.out_flags[b] |= extra;
  }
}

// ---------------------------------------------------------------------------
// K4: full-row draws of untruncated rows.  Their S64 is not known (the row
// pass sums float exponentials only), so one pass over the sampled row takes
// four double sums per chunk:
//   ea = sum of e64_p(x)                     (summed over chunks: S64 of p)
//   eg = sum of e64_p(x) over x in G
//   qa = sum of q's unnormalised weight w_q(x): e64_q(x) for q formed from
//        the draft's logits (summed over chunks: S64 of q, Sq), the dense q
//        itself otherwise (used as given, Sq = 1)
//   qg = sum of w_q(x) over x in G
// where G = {x : p(x) > beta q(x)} is told apart with the float
// approximations of p and q (a term they could misplace differs from the
// cut by a few 1e-7 of its p, so its residual weight is of that order).
// A chunk's residual weight ([WR] §5: (p - q)_+) is eg / S64 - beta qg / Sq,
// its weight under p is ea; the token is then located by a rescan of the
// chunk holding the crossing of t = u * W, token by token with the same
// arithmetic.
// Two launches: big_partial_kernel (grid nch4 * B), workgroup ci of request
// b sums the tokens [2048 ci, 2048 ci + 2048) (thread t owns 8 consecutive
// tokens, 16-byte loads) in a fixed order; big_finish_kernel (grid B) forms
// the chunk weights, walks them and rescans.  Workgroups never wait on or
// signal each other inside a launch.
// ---------------------------------------------------------------------------
constexpr int kSeg = 8;  // tokens per thread segment
constexpr int kChunk4 = 256 * kSeg;

struct BigArgs {
  const void* logits;
  QSrc q;
  int64_t V;
  int32_t G1;
  int32_t nch4;
  double c64;
  const BigJob* jobs;
  double* partials;  // [B][nch4][4]: ea, eg, qa, qg
  int32_t* out_tokens;
  uint32_t* out_flags;
  int32_t eos;       // end-of-sequence id, < 0: none
  double beta;       // lenience (the residual is (p - beta q)_+)
};

// Raw logits and q values of tokens x0 .. x0+7 of the job's rows (-inf / q
// = 0 past V; 16-byte loads when aligned).
template <bool BF16>
__device__ __forceinline__ void seg_load(const BigArgs& a, const BigJob& jb, const QRow& qr, bool residual, int64_t x0,
                                         float* z, float* qv) {
  const int64_t V = a.V;
  const int64_t zo = (int64_t)jb.row * V + x0;
  const bool full = x0 + kSeg <= V;
  if constexpr (BF16) {
    if (full && (zo & 7) == 0) {
      widen<true>(reinterpret_cast<const uint4*>(a.logits)[zo >> 3], z);
    } else {
#pragma unroll
      for (int k = 0; k < kSeg; ++k) z[k] = (x0 + k < V) ? load_logit<true>(a.logits, zo + k) : kNegInf;
    }
  } else {
    if (full && (zo & 3) == 0) {
      const uint4* p = reinterpret_cast<const uint4*>(a.logits) + (zo >> 2);
      widen<false>(p[0], z);
      widen<false>(p[1], z + 4);
    } else {
#pragma unroll
      for (int k = 0; k < kSeg; ++k) z[k] = (x0 + k < V) ? load_logit<false>(a.logits, zo + k) : kNegInf;
    }
  }
  if (residual) qr.raw8(x0, V, qv);
}

// Per token of a segment: ep = e64_p, eq = w_q (residual only) and whether
// the token is in G.
__device__ __forceinline__ void seg_terms(const BigJob& jb, const QRow& qr, bool residual, double c64, double beta,
                                          const float* z, const float* qv, double* ep, double* eq, bool* gt) {
  const double invS = 1.0 / jb.S;
#pragma unroll
  for (int k = 0; k < kSeg; ++k) {
    ep[k] = (z[k] >= jb.tau) ? e64_of(z[k], c64, jb.R) : 0.0;
    eq[k] = 0.0;
    gt[k] = false;
    if (residual) {
      eq[k] = qr.e64raw(qv[k]);
      gt[k] = ep[k] * invS > beta * qr.approx(eq[k]);
    }
  }
}

// Weight of one token once the normalisers are known: the residual
// p - beta q on G (0 elsewhere), else e64_p.
__device__ __forceinline__ double term_weight(bool residual, double ep, double eq, bool gt, double invSp, double invSq,
                                              double beta) {
  if (!residual) return ep;
  return gt ? ep * invSp - beta * (eq * invSq) : 0.0;
}

// Sum of four values over a 256-thread workgroup in a fixed order; the
// totals land in s_out[0..3] (visible after the call's last barrier).
__device__ __forceinline__ void block_sum4(const double (&v)[4], double (*s_w)[4], double* s_out) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  double r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = wave_sum_d(v[i]);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s_w[wid][i] = r[i];
  }
  __syncthreads();
  if (tid < 4) s_out[tid] = ((s_w[0][tid] + s_w[1][tid]) + s_w[2][tid]) + s_w[3][tid];
  __syncthreads();
}

// Exclusive prefix of this thread's segment total within the chunk (threads
// in order), fixed order.
__device__ __forceinline__ double chunk_excl(double seg, double* s_w) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  double incl = wave_incl_scan_d(seg);
  const double ex = wave_prev_d(incl, 0.0);
  __syncthreads();
  if (lane == 63) s_w[wid] = incl;
  __syncthreads();
  double off = 0.0;
  for (int k = 0; k < wid; ++k) off += s_w[k];
  return off + ex;
}

// FUSED (untruncated rows, gamma + 1 <= 64): every workgroup of request b
// first takes the acceptance decision itself (wave 0; it is a few hundred
// bytes of reads, so repeating it per chunk is cheaper than a launch), chunk
// 0 writes the request's outputs and the job, then all sum their chunk.
template <bool BF16, bool FUSED>
__global__ void __launch_bounds__(256) big_partial_kernel(BigArgs a, AcceptArgs ac) {
  const int64_t blk = blockIdx.x;
  const int b = (int)(blk / a.nch4), ci = (int)(blk - (int64_t)b * a.nch4);
  __shared__ double s_w[4][4];
  __shared__ double s_tot[4];
  __shared__ BigJob s_job;
  BigJob jb;
  if constexpr (FUSED) {
    const int lane = threadIdx.x & 63;
    if (threadIdx.x < kWave) {
      Decision dc = decide_short<BF16, true>(ac, b);
      const int P1 = ac.gamma + 1;
      int32_t* out = ac.out_tokens + (int64_t)b * P1;
      if (dc.bad) {
        if (ci == 0) empty_request(ac, b, out, dc.badfl);
        if (lane == 0) s_job.active = 0;
      } else if (dc.eos_cut) {
        if (ci == 0) finish_request<BF16>(ac, b, dc, out);  // no draw
        if (lane == 0) s_job.active = 0;
      } else {
        const bool residual = dc.nacc < dc.G;
        if (lane == 0) {
          BigJob j;
          j.S = dc.rs.S;
          j.S64 = 0.0;
          j.R = dc.rs.R;
          j.tau = dc.rs.tau;
          j.u = ac.ur[(int64_t)dc.lo + b + dc.nacc];
          j.row = (int32_t)((int64_t)dc.lo + b + dc.nacc);
          j.qrow = residual ? (int32_t)(dc.lo + dc.nacc) : -1;
          j.slot = dc.nacc;
          j.active = 1;
          j.pad = 0;
          s_job = j;
        }
        if (ci == 0) {
          for (int jj = lane; jj < P1; jj += kWave)
            if (jj != dc.nacc) out[jj] = jj < dc.nacc ? ac.ids[(int64_t)dc.lo + jj] : -1;
          if (lane == 0) {
            ac.out_nacc[b] = dc.nacc;
            if (ac.out_flags) ac.out_flags[b] = dc.fl;
            ac.jobs[b] = s_job;
          }
        }
      }
    }
    __syncthreads();
    jb = s_job;
  } else {
    jb = a.jobs[b];
  }
  if (!jb.active) return;
  const bool res = jb.qrow >= 0;
  const QRow qr = res ? q_row(a.q, jb.qrow) : q_none();
  const int64_t x0 = (int64_t)ci * kChunk4 + (int64_t)threadIdx.x * kSeg;
  float z[kSeg], qv[kSeg];
  seg_load<BF16>(a, jb, qr, res, x0, z, qv);
  double ep[kSeg], eq[kSeg];
  bool gt[kSeg];
  seg_terms(jb, qr, res, a.c64, a.beta, z, qv, ep, eq, gt);
  double v[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int k = 0; k < kSeg; ++k) {
    v[0] += ep[k];
    v[2] += eq[k];
    if (gt[k]) {
      v[1] += ep[k];
      v[3] += eq[k];
    }
  }
  block_sum4(v, s_w, s_tot);
  if (threadIdx.x < 4) a.partials[((int64_t)b * a.nch4 + ci) * 4 + threadIdx.x] = s_tot[threadIdx.x];
}

// One workgroup per request: the normalisers and chunk weights from the
// chunk sums (written by the previous launch), the walk to the chunk that
// holds the token, and its rescan.
template <bool BF16>
__global__ void __launch_bounds__(256) big_finish_kernel(BigArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int b = blockIdx.x;
  const double* P = a.partials + (int64_t)b * a.nch4 * 4;
  // rows of at most 64 chunks: wave 0 loads lane k's four chunk sums
  // together with the job (the address does not depend on it)
  const bool few = a.nch4 <= kWave;
  double cs[4] = {0.0, 0.0, 0.0, 0.0};
  if (few && wid == 0 && lane < a.nch4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) cs[i] = P[lane * 4 + i];
  }
  const BigJob jb = a.jobs[b];
  if (!jb.active) return;
  __shared__ double s_w[4];
  __shared__ int s_cstar, s_wf[4], s_wl[4];
  __shared__ double s_carry, s_t, s_inv[2];
  __shared__ int s_res;
  bool residual = jb.qrow >= 0;
  const bool qlog = residual && a.q.dense == nullptr && a.q.z != nullptr;
  uint32_t extra = 0;
  if (wid == 0) {
    // normalisers: chunk sums in a fixed order (lanes over chunks, then the
    // wave reduction)
    double sp = 0.0, sq = 0.0;
    if (few) {
      sp += cs[0];
      sq += cs[2];
    } else {
      for (int k = lane; k < a.nch4; k += kWave) {
        sp += P[k * 4 + 0];
        sq += P[k * 4 + 2];
      }
    }
    sp = wave_sum_d(sp);
    sq = wave_sum_d(sq);
    const double invSp = 1.0 / sp, invSq = qlog ? 1.0 / sq : 1.0;
    auto wchunk = [&](int k, bool res) -> double {
      if (k >= a.nch4) return 0.0;
      if (few) return res ? cs[1] * invSp - a.beta * (cs[3] * invSq) : cs[0];  // k == lane
      return res ? P[k * 4 + 1] * invSp - a.beta * (P[k * 4 + 3] * invSq) : P[k * 4 + 0];
    };
    // total weight (the same scans as the walk below: identical sums)
    auto walk_total = [&](bool res) {
      double carry = 0.0;
      for (int k0 = 0; k0 < a.nch4; k0 += kWave) {
        const double incl = wave_incl_scan_d(wchunk(k0 + lane, res));
        carry = carry + wave_last_d(incl);
      }
      return carry;
    };
    double tot = walk_total(residual);
    if (residual && !(tot > 0.0)) {
      extra |= 4u;  // SV_ROW_Z_DEGENERATE: draw from p instead
      residual = false;
      tot = walk_total(false);
    }
    const double t = (double)jb.u * tot;
    double carry = 0.0;
    int cstar = -1, lastc = -1;
    double cex = 0.0;
    for (int k0 = 0; k0 < a.nch4; k0 += kWave) {
      const int k = k0 + lane;
      const double pk = wchunk(k, residual);
      const double incl = wave_incl_scan_d(pk);
      const double C = carry + incl;
      const double ex = wave_prev_d(C, carry);
      const uint64_t pos = ballot(k < a.nch4 && pk > 0.0);
      if (pos) lastc = k0 + 63 - (int)__builtin_clzll(pos);
      const uint64_t hit = ballot(k < a.nch4 && C > t);
      if (hit) {
        const int src = (int)__builtin_ctzll(hit);
        cstar = k0 + src;
        cex = __shfl(ex, src, kWave);
        break;
      }
      carry = carry + wave_last_d(incl);
    }
    if (cstar < 0) {
      // rounding left no chunk above t: the last positive token of the last
      // positive chunk
      cstar = lastc;
      cex = -1.0 / 0.0;
    }
    if (lane == 0) {
      s_cstar = cstar;
      s_carry = cex;
      s_t = t;
      s_inv[0] = invSp;
      s_inv[1] = invSq;
      s_res = residual ? 1 : 0;
    }
  }
  __syncthreads();
  const int cstar = s_cstar;
  residual = s_res != 0;
  int token = -1;
  if (cstar >= 0) {
    const double t = s_t, invSp = s_inv[0], invSq = s_inv[1];
    const QRow qr = residual ? q_row(a.q, jb.qrow) : q_none();
    const int64_t x0 = (int64_t)cstar * kChunk4 + (int64_t)tid * kSeg;
    float z[kSeg], qv[kSeg];
    seg_load<BF16>(a, jb, qr, residual, x0, z, qv);
    double ep[kSeg], eq[kSeg], w[kSeg];
    bool gt[kSeg];
    seg_terms(jb, qr, residual, a.c64, a.beta, z, qv, ep, eq, gt);
    double seg = 0.0;
#pragma unroll
    for (int k = 0; k < kSeg; ++k) {
      w[k] = term_weight(residual, ep[k], eq[k], gt[k], invSp, invSq, a.beta);
      seg += w[k];
    }
    double run = s_carry + chunk_excl(seg, s_w);
    int found = 0x7fffffff, lp = -1;
#pragma unroll
    for (int k = 0; k < kSeg; ++k) {
      run = run + w[k];
      if (w[k] > 0.0) lp = (int)(x0 + k);
      if (run > t && found == 0x7fffffff) found = (int)(x0 + k);
    }
    token = block_first_or_last<4>(found, lp, s_wf, s_wl);
  }
  if (tid == 0) {
    a.out_tokens[(int64_t)b * a.G1 + jb.slot] = token;
    if (a.eos >= 0 && token == a.eos) extra |= 16u;  // SV_ROW_EOS
    if (extra && a.out_flags) a.out_flags[b] |= extra;
  }
}

// ---------------------------------------------------------------------------
// Untruncated requests with gamma + 1 <= 64, in one launch: one workgroup
// of BS threads per request takes the acceptance decision (wave 0), sums the
// sampled row in tiles of BS * 8 tokens (each thread 8 consecutive tokens,
// 16-byte loads; the four sums of K4 per tile, reduced in a fixed order and
// kept in LDS), then re-weighs only the tile holding t = u * W (now in L2)
// to find the token.
// ---------------------------------------------------------------------------
constexpr int kMaxTiles = 64;  // rows up to 64 * 8192 tokens (BS = 1024)

template <int BS>
__device__ __forceinline__ double block_excl_scan(double v, double& total, double* s_wt) {
  constexpr int NW = BS / kWave;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  double incl = wave_incl_scan_d(v);
  const double ex = wave_prev_d(incl, 0.0);
  __syncthreads();
  if (lane == 63) s_wt[wid] = incl;
  __syncthreads();
  double off = 0.0;
  for (int k = 0; k < wid; ++k) off += s_wt[k];
  double tot = 0.0;
  for (int k = 0; k < NW; ++k) tot += s_wt[k];
  total = tot;
  return off + ex;
}

template <bool BF16, int BS>
__global__ void __launch_bounds__(BS) sample_full_kernel(BigArgs a, AcceptArgs ac) {
  constexpr int NW = BS / kWave;
  constexpr int kU = BS >= 1024 ? 2 : 4;  // tiles whose loads are in flight together (128 VGPRs at 1024 threads)
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int b = blockIdx.x;
  __shared__ BigJob s_job;
  __shared__ double s_wt[NW];
  __shared__ double s_part[4][kMaxTiles * NW];  // per-wave tile sums (ea, eg, qa, qg)
  __shared__ double s_tile[4][kMaxTiles];
  __shared__ int s_kstar, s_wf[NW], s_wl[NW], s_res;
  __shared__ double s_cex, s_t, s_inv[2];
  const int P1 = ac.gamma + 1;
  int32_t* out = ac.out_tokens + (int64_t)b * P1;
  if (tid < kWave) {
    Decision dc = decide_short<BF16, true>(ac, b);
    if (dc.bad) {
      empty_request(ac, b, out, dc.badfl);
      if (lane == 0) s_job.active = 0;
    } else if (dc.eos_cut) {
      finish_request<BF16>(ac, b, dc, out);  // no draw
      if (lane == 0) s_job.active = 0;
    } else {
      const bool residual = dc.nacc < dc.G;
      for (int jj = lane; jj < P1; jj += kWave)
        if (jj != dc.nacc) out[jj] = jj < dc.nacc ? ac.ids[(int64_t)dc.lo + jj] : -1;
      if (lane == 0) {
        BigJob j;
        j.S = dc.rs.S;
        j.S64 = 0.0;
        j.R = dc.rs.R;
        j.tau = dc.rs.tau;
        j.u = ac.ur[(int64_t)dc.lo + b + dc.nacc];
        j.row = (int32_t)((int64_t)dc.lo + b + dc.nacc);
        j.qrow = residual ? (int32_t)(dc.lo + dc.nacc) : -1;
        j.slot = dc.nacc;
        j.active = 1;
        j.pad = (int32_t)dc.fl;
        s_job = j;
        ac.out_nacc[b] = dc.nacc;
      }
    }
  }
  __syncthreads();
  const BigJob jb = s_job;
  if (!jb.active) return;
  uint32_t fl = (uint32_t)jb.pad;
  bool residual = jb.qrow >= 0;
  const bool qlog = residual && a.q.dense == nullptr && a.q.z != nullptr;
  const QRow qr = residual ? q_row(a.q, jb.qrow) : q_none();
  constexpr int64_t kTileN = (int64_t)BS * kSeg;
  const int ntiles = (int)((a.V + kTileN - 1) / kTileN);

  // Pass 1: tile sums.  Loads of kU tiles are issued together; each wave
  // reduces its share of a tile and parks it in LDS (no barrier in the loop).
  for (int k0 = 0; k0 < ntiles; k0 += kU) {
    float z[kU][kSeg], qv[kU][kSeg];
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (k0 + u < ntiles)
        seg_load<BF16>(a, jb, qr, residual, (int64_t)(k0 + u) * kTileN + (int64_t)tid * kSeg, z[u], qv[u]);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (k0 + u >= ntiles) break;
      double ep[kSeg], eq[kSeg];
      bool gt[kSeg];
      seg_terms(jb, qr, residual, a.c64, a.beta, z[u], qv[u], ep, eq, gt);
      double v[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int i = 0; i < kSeg; ++i) {
        v[0] += ep[i];
        v[2] += eq[i];
        if (gt[i]) {
          v[1] += ep[i];
          v[3] += eq[i];
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double ws = wave_sum_d(v[i]);
        if (lane == 0) s_part[i][(k0 + u) * NW + wid] = ws;
      }
    }
  }
  __syncthreads();
  for (int k = tid; k < 4 * ntiles; k += BS) {
    const int i = k / ntiles, kt = k - i * ntiles;
    double t = 0.0;
    for (int w2 = 0; w2 < NW; ++w2) t += s_part[i][kt * NW + w2];
    s_tile[i][kt] = t;
  }
  __syncthreads();
  if (tid == 0) {
    double sp = 0.0, sq = 0.0;
    for (int k = 0; k < ntiles; ++k) {
      sp += s_tile[0][k];
      sq += s_tile[2][k];
    }
    const double invSp = 1.0 / sp, invSq = qlog ? 1.0 / sq : 1.0;
    auto wtile = [&](int k, bool res) {
      return res ? s_tile[1][k] * invSp - a.beta * (s_tile[3][k] * invSq) : s_tile[0][k];
    };
    double W = 0.0;
    for (int k = 0; k < ntiles; ++k) W = W + wtile(k, residual);
    if (residual && !(W > 0.0)) {
      fl |= 4u;  // SV_ROW_Z_DEGENERATE: draw from p instead
      residual = false;
      W = 0.0;
      for (int k = 0; k < ntiles; ++k) W = W + wtile(k, false);
    }
    const double t = (double)jb.u * W;
    double carry = 0.0;
    int kstar = -1, lastk = -1;
    for (int k = 0; k < ntiles; ++k) {
      const double tk = wtile(k, residual);
      if (tk > 0.0) lastk = k;
      if (carry + tk > t) {
        kstar = k;
        break;
      }
      carry = carry + tk;
    }
    if (kstar < 0) {
      // rounding left no tile above t: the last positive token of the last
      // positive tile
      kstar = lastk;
      carry = -1.0 / 0.0;
    }
    s_kstar = kstar;
    s_cex = carry;
    s_t = t;
    s_inv[0] = invSp;
    s_inv[1] = invSq;
    s_res = residual ? 1 : 0;
  }
  __syncthreads();
  const int kstar = s_kstar;
  residual = s_res != 0;
  int token = -1;
  if (kstar >= 0) {
    const double invSp = s_inv[0], invSq = s_inv[1];
    const int64_t x0 = (int64_t)kstar * kTileN + (int64_t)tid * kSeg;
    float z[kSeg], qv[kSeg];
    seg_load<BF16>(a, jb, qr, residual, x0, z, qv);
    double ep[kSeg], eq[kSeg], w[kSeg];
    bool gt[kSeg];
    seg_terms(jb, qr, residual, a.c64, a.beta, z, qv, ep, eq, gt);
    double seg = 0.0;
#pragma unroll
    for (int i = 0; i < kSeg; ++i) {
      w[i] = term_weight(residual, ep[i], eq[i], gt[i], invSp, invSq, a.beta);
      seg += w[i];
    }
    double tot;
    const double ex = block_excl_scan<BS>(seg, tot, s_wt);
    const double t = s_t;
    double run = s_cex + ex;
    int found = 0x7fffffff, lp = -1;
#pragma unroll
    for (int i = 0; i < kSeg; ++i) {
      run = run + w[i];
      if (w[i] > 0.0) lp = (int)(x0 + i);
      if (run > t && found == 0x7fffffff) found = (int)(x0 + i);
    }
    token = block_first_or_last<NW>(found, lp, s_wf, s_wl);
  }
  if (tid == 0) {
    if (ac.eos >= 0 && token == ac.eos) fl |= 16u;  // SV_ROW_EOS
    out[jb.slot] = token;
    if (ac.out_flags) ac.out_flags[b] = fl;
  }
}

// ---------------------------------------------------------------------------
// Greedy ([WR] §7.1): one wave per request merges the chunk argmaxes of its
// gamma+1 rows and finds the first mismatch.
// ---------------------------------------------------------------------------
struct GreedyArgs {
  const ChunkOut* cout;
  int32_t nchunks;
  const int32_t* ids;
  int32_t B;
  int32_t gamma;        // (maximum) drafts per request
  int64_t V;
  int32_t* out_tokens;  // [B, gamma + 1]
  int32_t* out_nacc;
  uint32_t* out_flags;
  const int32_t* cu;    // ragged draft offsets [B + 1], or null (Layout)
  int32_t n_draft;
  int32_t eos;          // end-of-sequence id, < 0: none
};

__global__ void __launch_bounds__(256) greedy_kernel(GreedyArgs a) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int b = blockIdx.x * 4 + wid;
  if (b >= a.B) return;
  const int P1 = a.gamma + 1;
  int32_t* out = a.out_tokens + (int64_t)b * P1;
  const Span sp = span_of(Layout{a.cu, a.n_draft, a.gamma}, b);
  if (!sp.ok) {
    for (int jj = lane; jj < P1; jj += kWave) out[jj] = -1;
    if (lane == 0) {
      a.out_nacc[b] = 0;
      if (a.out_flags) a.out_flags[b] = 32u;  // SV_ROW_BAD_SPAN
    }
    return;
  }
  const int G = sp.g;
  const int64_t lo = sp.lo;
  if (P1 <= kWave) {
    // Row j's argmax from its chunk results: L lanes per row (L a power of
    // two, L * (gamma + 1) <= 64) take every L-th chunk, all loads in flight
    // together, and meet by xor shuffles inside their group; the (max, lowest
    // id) merge does not depend on the order of the chunks.  Lane j then
    // holds row j, and the first mismatch comes by ballot.
    int L = 1;
    while (L * 2 * P1 <= kWave) L *= 2;
    const int jr = lane / L, t = lane & (L - 1);
    float v = kNegInf;
    int i = 0x7fffffff, d = -1;
    uint32_t fl = 0;
    if (lane < G) d = a.ids[lo + lane];
    if (jr <= G) {
      const ChunkOut* co = a.cout + (lo + b + jr) * a.nchunks;
      for (int c0 = t; c0 < a.nchunks; c0 += 8 * L) {
        ChunkOut o[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (c0 + k * L < a.nchunks) o[k] = co[c0 + k * L];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (c0 + k * L >= a.nchunks) break;
          argmax_merge(v, i, o[k].xmax, o[k].argmax);
          fl |= o[k].flags;
        }
      }
    }
    for (int o = 1; o < L; o <<= 1) {
      const float v2 = __shfl_xor(v, o, kWave);
      const int i2 = __shfl_xor(i, o, kWave);
      fl |= (uint32_t)__shfl_xor((int)fl, o, kWave);
      argmax_merge(v, i, v2, i2);
    }
    const int src = (lane < P1 ? lane : 0) * L;
    v = __shfl(v, src, kWave);
    i = __shfl(i, src, kWave);
    fl = (uint32_t)__shfl((int)fl, src, kWave);
    if (lane > G) fl = 0;
    if (ballot(lane <= G && (fl & CF_NAN)) != 0) {
      if (lane < P1) out[lane] = -1;
      if (lane == 0) {
        a.out_nacc[b] = 0;
        if (a.out_flags) a.out_flags[b] = 8u;  // SV_ROW_NONFINITE
      }
      return;
    }
    const uint64_t mism = ballot(lane < G && d != i);
    int n = mism ? (int)__builtin_ctzll(mism) : G;
    bool eos_cut = false;
    if (a.eos >= 0) {
      // an accepted end of sequence ends the output ([WR] §14.3)
      const uint64_t em = ballot(lane < n && d == a.eos);
      if (em) {
        n = (int)__builtin_ctzll(em);
        eos_cut = true;
      }
    }
    const int gn = eos_cut ? a.eos : __shfl(i, n, kWave);
    const int dn = __shfl(d, n, kWave);
    if (lane < P1) out[lane] = lane < n ? d : (lane == n ? gn : -1);
    if (lane == 0) {
      a.out_nacc[b] = n;
      uint32_t f = 0;
      if (n < G && !eos_cut && (dn < 0 || (int64_t)dn >= a.V)) f |= 1u;  // SV_ROW_BAD_ID
      if (a.eos >= 0 && gn == a.eos) f |= 16u;                          // SV_ROW_EOS
      if (a.out_flags) a.out_flags[b] = f;
    }
    return;
  }
  // long drafts: row by row
  bool nan_any = false;
  int n = G, gn = -1;
  bool decided = false, eos_cut = false;
  for (int jj = 0; jj <= G; ++jj) {
    const ChunkOut* co = a.cout + (lo + b + jj) * a.nchunks;
    float v = kNegInf;
    int i = 0x7fffffff;
    uint32_t fl = 0;
    for (int c = lane; c < a.nchunks; c += kWave) {
      ChunkOut o = co[c];
      argmax_merge(v, i, o.xmax, o.argmax);
      fl |= o.flags;
    }
    wave_argmax(v, i);
    fl = wave_or(fl);
    if (fl & CF_NAN) nan_any = true;
    if (!decided) {
      if (jj == G) {
        gn = i;
        decided = true;
      } else {
        int d = a.ids[lo + jj];
        if (d != i) {
          n = jj;
          gn = i;
          decided = true;
        } else if (a.eos >= 0 && d == a.eos) {
          // an accepted end of sequence ends the output ([WR] §14.3)
          n = jj;
          gn = d;
          decided = true;
          eos_cut = true;
        }
      }
    }
  }
  if (nan_any) {
    for (int jj = lane; jj < P1; jj += kWave) out[jj] = -1;
    if (lane == 0) {
      a.out_nacc[b] = 0;
      if (a.out_flags) a.out_flags[b] = 8u;
    }
    return;
  }
  for (int jj = lane; jj < P1; jj += kWave) out[jj] = jj < n ? a.ids[lo + jj] : (jj == n ? gn : -1);
  if (lane == 0) {
    a.out_nacc[b] = n;
    uint32_t fl = 0;
    if (n < G && !eos_cut) {
      int d = a.ids[lo + n];
      if (d < 0 || (int64_t)d >= a.V) fl |= 1u;
    }
    if (a.eos >= 0 && gn == a.eos) fl |= 16u;  // SV_ROW_EOS
    if (a.out_flags) a.out_flags[b] = fl;
  }
}

// ---------------------------------------------------------------------------
// Statistics ([WR] §4.2, [RL] §2, [BS] §五): alpha = sum min(p, q),
// Z = sum (p - q)_+, Z' = sum (q - p)_+ and a = min(1, p(d) / q(d)) per
// position, every p (and a q formed from the draft's logits) in double:
// p = e64 / S64.
//   Rows whose kept set is a stored list (truncated rows): p is 0 off the
//     list, so alpha and Z are sums over the list; Z' adds, for a dense q,
//     sum(q) over the row minus its sum over the list (qsum_kernel sums q
//     beside the other kernels, only when Z' is asked for, and
//     stats_zqp_kernel completes Z' once it is in), and for q formed from
//     the draft's logits it is the sum over q's own list with p evaluated
//     at its ids.
//   Other rows stream the logits and q together, chunk by chunk, into the
//     three sums of the plain definitions, term by term: min(p, q),
//     (p - q)_+ and (q - p)_+, each p (and a q formed from the draft's
//     logits) a true division e64 / S64.  A truncated row carries its S64;
//     an untruncated row's S64 is summed first, by s64_chunk_kernel, so
//     that every term is classified by its p and q in double, as the
//     definitions do: a sign taken from float approximations misplaces the
//     terms where p and q agree to a few 1e-7, which moves a small Z by as
//     much.
// Each output may be null (not written).
// ---------------------------------------------------------------------------
struct StatsArgs {
  const void* logits;
  QSrc q;
  const Cand* qkept;    // q's kept lists [B * gamma][kmax] (q from logits, truncated rows), else null
  const int32_t* ids;
  int64_t V;
  int32_t gamma;
  int32_t nchunks;
  int64_t chunk;
  double c64;
  // Row results of the target's rows 0..gamma-1: info and kept lists of
  // position j of request b at row b * info_rpr + j (info_rpr = gamma for
  // the statistics call's own row passes, gamma + 1 when they are the
  // sampling call's).
  const RowInfo* info;
  const Cand* kept;
  int32_t info_rpr;
  int32_t kmax;
  // Untruncated rows' S64 as chunk sums [B * gamma][s64_nch] (s64_chunk_kernel):
  const double* p_s64;  // the target's rows (else null)
  const double* q_s64;  // the draft's rows, q from the draft's logits (else null)
  int32_t s64_nch;
  double* partials;     // [rows][nchunks][kStatSums]
  const double* qsum;   // dense q's row sums by chunk [rows][nchq] (qsum_kernel), for Z'
  int32_t nchq;
  // Listed rows with a dense q, Z' asked for: the finish stores the list's
  // two sums here [rows][2] (sum of q, sum of (q - p)_+ over the list), and
  // stats_zqp_kernel completes Z' once the q sums are in; null: the finish
  // reads the q sums itself.
  double* zqp_part;
  float* out_alpha;
  float* out_zpq;
  float* out_zqp;
  float* out_acc;
  int64_t rows;
};

// The sums of a streamed row: min(p, q), (p - q)_+ and (q - p)_+.
enum { ST_MIN = 0, ST_PQ = 1, ST_QP = 2, kStatSums = 3 };

// S64 of an untruncated row from its chunk sums, added in one fixed order
// (lane-strided, then the wave reduction), so that every wave that asks
// gets the same double.  Called by whole waves.
__device__ __forceinline__ double row_s64(const double* part, int64_t r, int nch) {
  double v = 0.0;
  for (int c = threadIdx.x & 63; c < nch; c += kWave) v += part[r * nch + c];
  return wave_sum_d(v);
}

// S64 of the target's row r: its own where the row carries one (truncated
// rows), else the sum of its chunk sums.
__device__ __forceinline__ double stats_s64_p(const StatsArgs& a, const RowInfo& ri, int64_t r) {
  return (ri.S64 > 0.0 || a.p_s64 == nullptr) ? ri.S64 : row_s64(a.p_s64, r, a.s64_nch);
}

// q's row r, with the S64 of an untruncated draft row filled in.
__device__ __forceinline__ QRow stats_q_row(const StatsArgs& a, int64_t r) {
  QRow qr = q_row(a.q, r);
  if (qr.logits_src() && !(qr.S64 > 0.0) && a.q_s64 != nullptr) qr.S64 = row_s64(a.q_s64, r, a.s64_nch);
  return qr;
}

// S64 of untruncated rows, by chunks: workgroup c of statistics row r sums
// e64 over [c * chunk, (c + 1) * chunk) of the row, each thread its 8-token
// segments in order, then a fixed-order workgroup sum.  The rows are the
// target's (logits [B][gamma + 1][V], row results at info rows
// b * info_rpr + j) or the draft's (logits [B][gamma][V], info_rpr = gamma).
struct S64Args {
  const void* logits;
  const RowInfo* info;
  int64_t V;
  int32_t gamma;
  int32_t lrpr;      // logits rows per request
  int32_t info_rpr;  // row results per request
  int32_t nchunks;
  int64_t chunk;
  double c64;
  double* out;       // [B * gamma][nchunks]
};

template <bool BF16>
__global__ void __launch_bounds__(256) s64_chunk_kernel(S64Args a) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t blk = blockIdx.x;
  const int64_t r = blk / a.nchunks;
  const int ci = (int)(blk - r * a.nchunks);
  const int64_t b = r / a.gamma, j = r - b * a.gamma;
  const RowInfo ri = a.info[b * a.info_rpr + j];
  const int64_t lrow = (b * a.lrpr + j) * a.V;
  const int64_t x0 = (int64_t)ci * a.chunk, x1 = min(x0 + a.chunk, a.V);
  __shared__ double s_w[4];
  // rows whose statistics are NaN (non-finite logits) are not read
  if (ri.flags & RF_NONFINITE) return;
  const bool vec = (a.V & 7) == 0;  // rows (and chunks) 16-byte aligned
  double acc = 0.0;
  constexpr int kU = 2;
  for (int64_t x = x0 + (int64_t)tid * 8; x < x1; x += (int64_t)kU * 256 * 8) {
    float z[kU][8];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t xu = x + (int64_t)u * 256 * 8;
      if (vec && xu + 8 <= x1) {
        if constexpr (BF16) {
          widen<true>(*reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.logits) + lrow + xu), z[u]);
        } else {
          const uint4* p4 = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(a.logits) + lrow + xu);
          widen<false>(p4[0], z[u]);
          widen<false>(p4[1], z[u] + 4);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) z[u][k] = xu + k < x1 ? load_logit<BF16>(a.logits, lrow + xu + k) : kNegInf;
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc += e64_of(z[u][k], a.c64, ri.R);
  }
  acc = wave_sum_d(acc);
  if (lane == 0) s_w[wid] = acc;
  __syncthreads();
  if (tid == 0) a.out[r * a.nchunks + ci] = ((s_w[0] + s_w[1]) + s_w[2]) + s_w[3];
}

__device__ __forceinline__ int64_t info_row(const StatsArgs& a, int64_t r) {
  const int64_t b = r / a.gamma;
  return b * a.info_rpr + (r - b * a.gamma);
}

// Does the row need the full-row sums of the chunk pass?
__device__ __forceinline__ bool stats_streamed(const StatsArgs& a, const RowInfo& ri, int64_t r) {
  if (a.q.dense != nullptr) return (ri.flags & RF_BIG) != 0;
  return ((ri.flags | a.q.info[r].flags) & RF_BIG) != 0 || a.qkept == nullptr;
}

// Sum of a dense q over each of its rows, for Z' of rows whose p is a kept
// list (Z' = sum q - sum over the list of q + sum over the list of
// (q - p)+).  It reads nothing but q, so it runs beside the target's passes
// (the statistics finish waits for it).  Workgroup c of row r sums the
// kQSumChunk floats [c * kQSumChunk, ...) of the row: each thread eight
// 16-byte segments (non-temporal loads), all in flight at once, added in
// double in a fixed order.
constexpr int kQSumChunk = 256 * 32;  // floats per workgroup (32 KB)

struct QSumArgs {
  const float* q;   // [rows][V]
  int64_t V;
  int64_t rows;
  int32_t nchq;     // chunks per row
  double* out;      // [rows][nchq]
};

__global__ void __launch_bounds__(256) qsum_kernel(QSumArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t blk = blockIdx.x;
  const int64_t r = blk / a.nchq;
  const int c = (int)(blk - r * a.nchq);
  __shared__ double s_w[4];
  const int64_t x0 = (int64_t)c * kQSumChunk, x1 = min(x0 + (int64_t)kQSumChunk, a.V);
  const float* row = a.q + r * a.V;
  const bool vec = (a.V & 3) == 0;  // rows (and so segments of 4) 16-byte aligned
  constexpr int kSegs = kQSumChunk / (256 * 4);  // 16-byte segments per thread
  double acc = 0.0;
  uint4 w[kSegs];
#pragma unroll
  for (int k = 0; k < kSegs; ++k) {
    const int64_t x = x0 + ((int64_t)k * 256 + tid) * 4;
    if (vec && x + 4 <= x1) {
      w[k] = ld_stream(reinterpret_cast<const uint4*>(row + x));
    } else {
      float f[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = x + i < x1 ? row[x + i] : 0.0f;
      w[k] = make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
    }
  }
#pragma unroll
  for (int k = 0; k < kSegs; ++k) {
    acc += (double)__uint_as_float(w[k].x);
    acc += (double)__uint_as_float(w[k].y);
    acc += (double)__uint_as_float(w[k].z);
    acc += (double)__uint_as_float(w[k].w);
  }
  acc = wave_sum_d(acc);
  if (lane == 0) s_w[wid] = acc;
  __syncthreads();
  if (tid == 0) a.out[r * a.nchq + c] = ((s_w[0] + s_w[1]) + s_w[2]) + s_w[3];
}

// QLOG: q comes from the draft's logits (else dense).
template <bool BF16, bool QLOG>
__global__ void __launch_bounds__(256) stats_chunk_kernel(StatsArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t blk = blockIdx.x;
  const int64_t r = blk / a.nchunks;
  const int ci = (int)(blk - r * a.nchunks);
  const RowInfo ri = a.info[info_row(a, r)];
  const int b = (int)(r / a.gamma), j = (int)(r - (int64_t)b * a.gamma);
  const int64_t lrow = ((int64_t)b * (a.gamma + 1) + j) * a.V;
  const int64_t x0 = (int64_t)ci * a.chunk, x1 = min(x0 + a.chunk, a.V);
  double sm[kStatSums];
#pragma unroll
  for (int i = 0; i < kStatSums; ++i) sm[i] = 0.0;
  __shared__ double s_p[4][kStatSums];
  const bool big = stats_streamed(a, ri, r);
  // Rows finished from their lists skip the pass (a dense q's sum comes
  // from qsum_kernel); nothing reads their partials (the test is the same
  // for the whole workgroup).
  if ((ri.flags & RF_NONFINITE) || !big) return;
  const QRow qr = stats_q_row(a, r);
  const double S64 = stats_s64_p(a, ri, r);
  // rows are 16-byte aligned when V is a multiple of 8 (chunks are too)
  const bool vec = (a.V & 7) == 0;
  const int64_t ngroups = (x1 - x0 + 7) / 8;
  constexpr int kU = 2;
  for (int64_t g0 = 0; g0 < ngroups; g0 += (int64_t)kU * 256) {
    float qv[kU][8], zv[kU][8];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t x = x0 + (g0 + (int64_t)u * 256 + tid) * 8;
      if (vec && x + 8 <= x1) {
        qr.raw8_whole(x, qv[u]);
        if constexpr (BF16) {
          widen<true>(*reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.logits) + lrow + x), zv[u]);
        } else {
          const uint4* zp4 = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(a.logits) + lrow + x);
          widen<false>(zp4[0], zv[u]);
          widen<false>(zp4[1], zv[u] + 4);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const bool in = x + k < x1;
          qv[u][k] = in ? qr.raw_at(x + k) : (QLOG ? kNegInf : 0.0f);
          zv[u][k] = in ? load_logit<BF16>(a.logits, lrow + x + k) : kNegInf;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float z = zv[u][k];
        const double p = (z >= ri.tau) ? e64_of(z, a.c64, ri.R) / S64 : 0.0;
        const double q = qr.q64_div(qv[u][k]);
        const double d = p - q;
        sm[ST_MIN] += (p < q) ? p : q;
        if (d > 0.0) sm[ST_PQ] += d;
        if (d < 0.0) sm[ST_QP] -= d;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kStatSums; ++i) {
    const double v = wave_sum_d(sm[i]);
    if (lane == 0) s_p[wid][i] = v;
  }
  __syncthreads();
  if (tid < kStatSums) {
    double v = ((s_p[0][tid] + s_p[1][tid]) + s_p[2][tid]) + s_p[3][tid];
    a.partials[(r * a.nchunks + ci) * kStatSums + tid] = v;
  }
}

template <bool BF16>
__global__ void __launch_bounds__(256) stats_final_kernel(StatsArgs a) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * 4 + wid;
  if (r >= a.rows) return;
  const int64_t ir = info_row(a, r);
  const bool qlog = a.q.dense == nullptr;
  // The first kStatPre * 64 entries of p's kept list (and of q's, when its
  // Z' is asked for) are loaded together with the row info, before nkept
  // is known (a nucleus of a few hundred tokens then costs no round trip
  // but q at its ids); entries past nkept are never used.
  constexpr int kStatBlk = 8;
  constexpr int kStatPre = 4;
  const Cand* L = a.kept != nullptr ? a.kept + ir * a.kmax : nullptr;
  const Cand* Lq = (qlog && a.qkept != nullptr && a.out_zqp != nullptr) ? a.qkept + r * a.kmax : nullptr;
  Cand pre[kStatPre], qpre[kStatPre];
#pragma unroll
  for (int u = 0; u < kStatPre; ++u) {
    pre[u].v = 0.0f;
    pre[u].idx = 0;
    qpre[u] = pre[u];
    if (L != nullptr) pre[u] = L[lane + u * kWave];
    if (Lq != nullptr) qpre[u] = Lq[lane + u * kWave];
  }
  const RowInfo ri = a.info[ir];
  const float qnan = __builtin_nanf("");
  const bool qbad = qlog && (a.q.info[r].flags & RF_NONFINITE);
  if ((ri.flags & RF_NONFINITE) || qbad) {
    if (lane == 0) {
      if (a.out_alpha) a.out_alpha[r] = qnan;
      if (a.out_zpq) a.out_zpq[r] = qnan;
      if (a.out_zqp) a.out_zqp[r] = qnan;
      if (a.out_acc) a.out_acc[r] = qnan;
    }
    return;
  }
  const QRow qr = stats_q_row(a, r);
  const double S64 = stats_s64_p(a, ri, r);  // p = e64 / S64 by true division (see above)
  const int b = (int)(r / a.gamma), j = (int)(r - (int64_t)b * a.gamma);
  const int64_t lrow = ((int64_t)b * (a.gamma + 1) + j) * a.V;
  double alpha, zpq, zqp = 0.0;
  const bool has_d = ri.d >= 0;
  // the draft's q(d) in double: a dense q as given, else from the draft's logit
  const float qraw_d = (has_d && qlog) ? qr.raw_at(ri.d) : 0.0f;
  if (stats_streamed(a, ri, r)) {
    double sm[kStatSums];
#pragma unroll
    for (int i = 0; i < kStatSums; ++i) {
      double v = 0.0;
      for (int c = lane; c < a.nchunks; c += kWave) v += a.partials[(r * a.nchunks + c) * kStatSums + i];
      sm[i] = wave_sum_d(v);
    }
    alpha = sm[ST_MIN];
    zpq = sm[ST_PQ];
    zqp = sm[ST_QP];
  } else {
    // L: token-id order
    double mn = 0.0, pq = 0.0, qp = 0.0, sqk = 0.0;
    // kStatBlk list steps per round (a nucleus of a few hundred tokens in
    // one): their entry loads, then their q loads, are in flight together;
    // each lane still adds its entries in list order
    const int nk = ri.nkept;
    for (int i0 = lane; i0 < nk; i0 += kStatBlk * kWave) {
      Cand e[kStatBlk];
      float qf[kStatBlk];
      if (i0 == lane) {
#pragma unroll
        for (int u = 0; u < kStatBlk; ++u) {
          if (u < kStatPre) e[u] = pre[u];
          else if (i0 + u * kWave < nk) e[u] = L[i0 + u * kWave];
        }
      } else {
#pragma unroll
        for (int u = 0; u < kStatBlk; ++u)
          if (i0 + u * kWave < nk) e[u] = L[i0 + u * kWave];
      }
#pragma unroll
      for (int u = 0; u < kStatBlk; ++u) qf[u] = (i0 + u * kWave < nk) ? qr.raw_at(e[u].idx) : 0.0f;
#pragma unroll
      for (int u = 0; u < kStatBlk; ++u) {
        if (i0 + u * kWave >= nk) break;
        const double p = e64_of(e[u].v, a.c64, ri.R) / S64;
        const double qv = qr.q64_div(qf[u]);
        const double d = p - qv;
        mn += (p < qv) ? p : qv;
        if (d > 0.0) pq += d;
        if (d < 0.0) qp -= d;
        sqk += qv;
      }
    }
    alpha = wave_sum_d(mn);
    zpq = wave_sum_d(pq);
    qp = wave_sum_d(qp);
    sqk = wave_sum_d(sqk);
    if (a.out_zqp == nullptr) {
      // Z' not asked for: neither sum(q) nor q's list is read
    } else if (!qlog && a.zqp_part != nullptr) {
      // finished by stats_zqp_kernel after the q sums
      if (lane == 0) {
        a.zqp_part[2 * r] = sqk;
        a.zqp_part[2 * r + 1] = qp;
      }
    } else if (!qlog) {
      double sq = 0.0;
      for (int c = lane; c < a.nchq; c += kWave) sq += a.qsum[r * a.nchq + c];
      zqp = (wave_sum_d(sq) - sqk) + qp;
    } else {
      // Z' = sum over q's kept set of (q - p)_+, with p read at its ids
      const RowInfo qi = a.q.info[r];
      const double qS64 = qi.S64;
      double zq = 0.0;
      const int nq = qi.nkept;
      for (int i0 = lane; i0 < nq; i0 += kStatBlk * kWave) {
        Cand e[kStatBlk];
        float zf[kStatBlk];
        if (i0 == lane) {
#pragma unroll
          for (int u = 0; u < kStatBlk; ++u) {
            if (u < kStatPre) e[u] = qpre[u];
            else if (i0 + u * kWave < nq) e[u] = Lq[i0 + u * kWave];
          }
        } else {
#pragma unroll
          for (int u = 0; u < kStatBlk; ++u)
            if (i0 + u * kWave < nq) e[u] = Lq[i0 + u * kWave];
        }
#pragma unroll
        for (int u = 0; u < kStatBlk; ++u)
          zf[u] = (i0 + u * kWave < nq) ? load_logit<BF16>(a.logits, lrow + e[u].idx) : kNegInf;
#pragma unroll
        for (int u = 0; u < kStatBlk; ++u) {
          if (i0 + u * kWave >= nq) break;
          const double qv = e64_of(e[u].v, a.c64, qi.R) / qS64;
          const float z = zf[u];
          const double p = (z >= ri.tau) ? e64_of(z, a.c64, ri.R) / S64 : 0.0;
          if (qv > p) zq += qv - p;
        }
      }
      zqp = wave_sum_d(zq);
    }
  }
  const bool deferred_zqp = !stats_streamed(a, ri, r) && !qlog && a.zqp_part != nullptr;
  double pd = 0.0, qd = 0.0;
  if (has_d) {
    pd = (ri.zd >= ri.tau) ? e64_of(ri.zd, a.c64, ri.R) / S64 : 0.0;
    qd = qlog ? qr.q64_div(qraw_d) : (double)ri.qd;
  }
  if (lane == 0) {
    if (a.out_alpha) a.out_alpha[r] = (float)alpha;
    if (a.out_zpq) a.out_zpq[r] = (float)zpq;
    if (a.out_zqp && !(deferred_zqp)) a.out_zqp[r] = (float)zqp;
    float ap;
    if (!has_d) ap = qnan;
    else if (qd == 0.0) ap = pd > 0.0 ? 1.0f : 0.0f;
    else ap = (float)fmin(1.0, pd / qd);
    if (a.out_acc) a.out_acc[r] = ap;
  }
}

// Z' of listed rows with a dense q, once the q sums are in:
// Z' = (sum q - sum over the list of q) + sum over the list of (q - p)_+,
// the list's two sums from stats_final_kernel.  One wave per position;
// rows without a usable result (non-finite) or streamed were finished
// there.
__global__ void __launch_bounds__(256) stats_zqp_kernel(StatsArgs a) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * 4 + wid;
  if (r >= a.rows) return;
  const RowInfo ri = a.info[info_row(a, r)];
  if ((ri.flags & RF_NONFINITE) || stats_streamed(a, ri, r)) return;
  double sq = 0.0;
  for (int c = lane; c < a.nchq; c += kWave) sq += a.qsum[r * a.nchq + c];
  const double zqp = (wave_sum_d(sq) - a.zqp_part[2 * r]) + a.zqp_part[2 * r + 1];
  if (lane == 0) a.out_zqp[r] = (float)zqp;
}

}  // namespace sv
