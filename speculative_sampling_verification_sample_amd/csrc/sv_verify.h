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
// it leaves a BigJob for K4, which sums the weights of a whole row in chunks
// and lets the last chunk to finish locate the token.
#pragma once

#include "sv_device.h"
#include "sv_rowfinal.h"

namespace sv {

struct AcceptArgs {
  const RowInfo* info;  // [B * (gamma+1)]
  const Cand* kept;     // [rows][kmax]
  int32_t kmax;
  const float* q;
  const int32_t* ids;
  const float* ua;
  const float* ur;
  int32_t B;
  int32_t gamma;
  int64_t V;
  int32_t* out_tokens;
  int32_t* out_nacc;
  uint32_t* out_flags;  // may be null
  BigJob* jobs;
  uint32_t* counters;
};

// Draw from the kept list of one row (called by a whole wave).
// residual: weights (e/S - q)_+ on the list; otherwise e/S.
__device__ int draw_from_list(const Cand* L, int n, double S, const float* qrow, bool& residual, float u,
                              uint32_t& fl) {
  const int lane = lane_id();
  const double invS = 1.0 / S;
  auto weight = [&](int i, bool res) -> double {
    if (i >= n) return 0.0;
    Cand e = L[i];
    double p = (double)e.v * invS;
    if (!res) return p;
    double d = p - (double)qrow[e.idx];
    return d > 0.0 ? d : 0.0;
  };
  auto total = [&](bool res) -> double {
    double carry = 0.0;
    for (int i0 = 0; i0 < n; i0 += kWave) {
      double incl = wave_incl_scan_d(weight(i0 + lane, res));
      carry = carry + __shfl(incl, kWave - 1, kWave);
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
  for (int i0 = 0; i0 < n; i0 += kWave) {
    const int i = i0 + lane;
    const double w = weight(i, residual);
    const double incl = wave_incl_scan_d(w);
    const double C = carry + incl;
    uint64_t hit = ballot(i < n && C > t);
    if (hit) {
      token = L[i0 + (int)__builtin_ctzll(hit)].idx;
      break;
    }
    uint64_t pos = ballot(i < n && w > 0.0);
    if (pos) lastpos = L[i0 + 63 - (int)__builtin_clzll(pos)].idx;
    carry = carry + __shfl(incl, kWave - 1, kWave);
  }
  return token >= 0 ? token : lastpos;
}

__global__ void __launch_bounds__(256) accept_kernel(AcceptArgs a) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int b = blockIdx.x * 4 + wid;
  if (b >= a.B) return;
  const int G = a.gamma, G1 = G + 1;
  const RowInfo* inf = a.info + (int64_t)b * G1;
  int32_t* out = a.out_tokens + (int64_t)b * G1;

  bool bad = false;
  for (int jj = lane; jj <= G; jj += kWave) {
    RowInfo ri = inf[jj];
    if (ri.flags & RF_NONFINITE) bad = true;
    if (jj < G && ri.d >= 0 && !(ri.qd >= 0.0f && ri.qd < kPosInf)) bad = true;
  }
  if (ballot(bad) != 0) {
    for (int jj = lane; jj < G1; jj += kWave) out[jj] = -1;
    if (lane == 0) {
      a.out_nacc[b] = 0;
      if (a.out_flags) a.out_flags[b] = 8u;  // SV_ROW_NONFINITE
      a.jobs[b].active = 0;
    }
    return;
  }
  // acceptance scan
  int nacc = G;
  for (int j0 = 0; j0 < G; j0 += kWave) {
    const int jj = j0 + lane;
    bool acc = true;
    if (jj < G) {
      RowInfo ri = inf[jj];
      if (ri.d < 0) acc = false;
      else if (ri.qd == 0.0f) acc = ri.ed > 0.0f;
      else acc = (double)a.ua[(int64_t)b * G + jj] * (double)ri.qd * ri.S < (double)ri.ed;
    }
    uint64_t rej = ballot(!acc);
    if (rej) {
      nacc = j0 + (int)__builtin_ctzll(rej);
      break;
    }
  }
  uint32_t fl = 0;
  bool qz = false;
  for (int jj = lane; jj < min(nacc + 1, G); jj += kWave) {
    RowInfo ri = inf[jj];
    if (ri.d >= 0 && ri.qd == 0.0f) qz = true;
  }
  if (ballot(qz) != 0) fl |= 2u;  // SV_ROW_Q_ZERO
  if (nacc < G && inf[nacc].d == -2) fl |= 1u;  // SV_ROW_BAD_ID
  for (int jj = lane; jj < G1; jj += kWave)
    if (jj != nacc) out[jj] = jj < nacc ? a.ids[(int64_t)b * G + jj] : -1;

  const RowInfo rs = inf[nacc];
  bool residual = nacc < G;
  const float u = a.ur[(int64_t)b * G1 + nacc];
  const int64_t trow = (int64_t)b * G1 + nacc;
  const int64_t qrow = residual ? (int64_t)b * G + nacc : -1;
  if (rs.flags & RF_BIG) {
    if (lane == 0) {
      BigJob jb;
      jb.S = rs.S;
      jb.R = rs.R;
      jb.tau = rs.tau;
      jb.u = u;
      jb.row = (int32_t)trow;
      jb.qrow = (int32_t)qrow;
      jb.slot = nacc;
      jb.active = 1;
      jb.pad = 0;
      a.jobs[b] = jb;
      a.counters[b] = 0u;
      out[nacc] = -1;  // written by the full-row sampler
      a.out_nacc[b] = nacc;
      if (a.out_flags) a.out_flags[b] = fl;
    }
    return;
  }
  const float* qr = residual ? a.q + qrow * a.V : nullptr;
  int token = draw_from_list(a.kept + trow * a.kmax, rs.nkept, rs.S, qr, residual, u, fl);
  if (lane == 0) {
    out[nacc] = token;
    a.out_nacc[b] = nacc;
    if (a.out_flags) a.out_flags[b] = fl;
    a.jobs[b].active = 0;
  }
}

// ---------------------------------------------------------------------------
// K4: full-row draw.  Grid (nch4 * B); a workgroup sums the weights of one
// chunk of the sampled row in tiles (thread t owns `kSeg` consecutive
// elements of a tile), the last workgroup of a request to finish walks the
// chunk totals and rescans the chunk holding the token with the same
// arithmetic.
// ---------------------------------------------------------------------------
constexpr int kSeg = 16;
constexpr int kTile = 256 * kSeg;

struct BigArgs {
  const void* logits;
  const float* q;
  int64_t V;
  int32_t G1;
  int32_t nch4;
  int64_t ch4;  // multiple of kTile
  float c;
  const BigJob* jobs;
  uint32_t* counters;
  double* partials;  // [B][nch4]
  int32_t* out_tokens;
  uint32_t* out_flags;
};

template <bool BF16>
__device__ __forceinline__ double big_weight(const BigArgs& a, const BigJob& jb, bool residual, int64_t x) {
  float z = load_logit<BF16>(a.logits, (int64_t)jb.row * a.V + x);
  if (!(z >= jb.tau)) return 0.0;
  double e = (double)e_of(z, a.c, jb.R);
  if (!residual) return e;
  double d = e - (double)a.q[(int64_t)jb.qrow * a.V + x] * jb.S;
  return d > 0.0 ? d : 0.0;
}

// Weight total of tile [x0, x0 + kTile) ∩ [.., x1): per-thread segment sums
// and their exclusive scan (fixed order).  Returns the tile total.
template <bool BF16>
__device__ double tile_scan(const BigArgs& a, const BigJob& jb, bool residual, int64_t x0, int64_t x1,
                            double& seg, double& excl, double* s_w) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t s0 = x0 + (int64_t)tid * kSeg;
  double acc = 0.0;
  for (int k = 0; k < kSeg; ++k) {
    int64_t x = s0 + k;
    if (x < x1) acc += big_weight<BF16>(a, jb, residual, x);
  }
  seg = acc;
  double incl = wave_incl_scan_d(acc);
  __syncthreads();
  if (lane == 63) s_w[wid] = incl;
  __syncthreads();
  double off = 0.0;
  for (int w = 0; w < wid; ++w) off += s_w[w];
  excl = off + (incl - acc);
  double tot = ((s_w[0] + s_w[1]) + s_w[2]) + s_w[3];
  return tot;
}

template <bool BF16>
__device__ double chunk_total(const BigArgs& a, const BigJob& jb, bool residual, int64_t x0, int64_t x1,
                              double* s_w) {
  double tot = 0.0;
  for (int64_t t0 = x0; t0 < x1; t0 += kTile) {
    double seg, excl;
    tot = tot + tile_scan<BF16>(a, jb, residual, t0, x1, seg, excl, s_w);
  }
  return tot;
}

// Token in chunk [x0, x1) whose running weight (starting at `carry`) first
// exceeds t; the last positive-weight token of the chunk when rounding
// leaves none.
template <bool BF16>
__device__ int chunk_find(const BigArgs& a, const BigJob& jb, bool residual, int64_t x0, int64_t x1, double carry,
                          double t, double* s_w, int* s_best) {
  const int tid = threadIdx.x;
  int lastpos = -1;
  for (int64_t t0 = x0; t0 < x1; t0 += kTile) {
    double seg, excl;
    double tot = tile_scan<BF16>(a, jb, residual, t0, x1, seg, excl, s_w);
    if (tid == 0) {
      s_best[0] = 0x7fffffff;
      s_best[1] = -1;
    }
    __syncthreads();
    const int64_t s0 = t0 + (int64_t)tid * kSeg;
    double run = carry + excl;
    const bool here = carry + tot > t;
    int found = 0x7fffffff, lp = -1;
    for (int k = 0; k < kSeg; ++k) {
      int64_t x = s0 + k;
      if (x >= x1) break;
      double w = big_weight<BF16>(a, jb, residual, x);
      run = run + w;
      if (w > 0.0) lp = (int)x;
      if (here && run > t && found == 0x7fffffff) found = (int)x;
    }
    if (found != 0x7fffffff) atomicMin(&s_best[0], found);
    if (lp >= 0) atomicMax(&s_best[1], lp);
    __syncthreads();
    int f = s_best[0];
    if (s_best[1] >= 0) lastpos = s_best[1];
    __syncthreads();
    if (here) return f != 0x7fffffff ? f : lastpos;
    carry = carry + tot;
  }
  return lastpos;
}

template <bool BF16>
__global__ void __launch_bounds__(256) big_kernel(BigArgs a) {
  const int tid = threadIdx.x;
  const int64_t blk = blockIdx.x;
  const int b = (int)(blk / a.nch4), ci = (int)(blk - (int64_t)b * a.nch4);
  const BigJob jb = a.jobs[b];
  if (!jb.active) return;
  __shared__ double s_w[4];
  __shared__ int s_best[2];
  __shared__ int s_last;
  __shared__ int s_cstar;
  __shared__ double s_carry;
  bool residual = jb.qrow >= 0;
  const int64_t x0 = (int64_t)ci * a.ch4, x1 = min(x0 + a.ch4, a.V);
  double W = chunk_total<BF16>(a, jb, residual, x0, x1, s_w);
  double* P = a.partials + (int64_t)b * a.nch4;
  if (tid == 0) {
    P[ci] = W;
    __threadfence();
    unsigned old = atomicAdd(&a.counters[b], 1u);
    s_last = (old == (unsigned)(a.nch4 - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  uint32_t extra = 0;
  // total and chunk search (sequential, fixed order)
  auto locate = [&](double& tot_out) {
    if (tid == 0) {
      double tot = 0.0;
      for (int k = 0; k < a.nch4; ++k) tot = tot + __builtin_nontemporal_load(&P[k]);
      tot_out = tot;
      s_carry = tot;
    }
    __syncthreads();
    tot_out = s_carry;
    __syncthreads();
  };
  double tot;
  locate(tot);
  if (residual && !(tot > 0.0)) {
    extra |= 4u;  // SV_ROW_Z_DEGENERATE: draw from p instead
    residual = false;
    for (int k = 0; k < a.nch4; ++k) {
      const int64_t y0 = (int64_t)k * a.ch4, y1 = min(y0 + a.ch4, a.V);
      double wk = chunk_total<BF16>(a, jb, false, y0, y1, s_w);
      if (tid == 0) P[k] = wk;
    }
    __threadfence();
    __syncthreads();
    locate(tot);
  }
  const double t = (double)jb.u * tot;
  if (tid == 0) {
    double carry = 0.0;
    int cstar = -1, lastc = -1;
    for (int k = 0; k < a.nch4; ++k) {
      double pk = __builtin_nontemporal_load(&P[k]);
      if (pk > 0.0) lastc = k;
      if (carry + pk > t) {
        cstar = k;
        break;
      }
      carry = carry + pk;
    }
    if (cstar < 0) {
      // rounding left no chunk: the last positive token of the last
      // positive chunk (carry chosen so that nothing exceeds t)
      cstar = lastc;
      carry = -1.0 / 0.0;
    }
    s_cstar = cstar;
    s_carry = carry;
  }
  __syncthreads();
  const int cstar = s_cstar;
  const double carry = s_carry;
  int token = -1;
  if (cstar >= 0) {
    const int64_t y0 = (int64_t)cstar * a.ch4, y1 = min(y0 + a.ch4, a.V);
    token = chunk_find<BF16>(a, jb, residual, y0, y1, carry, t, s_w, s_best);
  }
  if (tid == 0) {
    a.out_tokens[(int64_t)b * a.G1 + jb.slot] = token;
    if (extra && a.out_flags) a.out_flags[b] |= extra;
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
  int32_t gamma;
  int64_t V;
  int32_t* out_tokens;
  int32_t* out_nacc;
  uint32_t* out_flags;
};

__global__ void __launch_bounds__(256) greedy_kernel(GreedyArgs a) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int b = blockIdx.x * 4 + wid;
  if (b >= a.B) return;
  const int G = a.gamma, G1 = G + 1;
  bool nan_any = false;
  int n = G, gn = -1;
  bool decided = false;
  for (int jj = 0; jj <= G; ++jj) {
    const ChunkOut* co = a.cout + ((int64_t)b * G1 + jj) * a.nchunks;
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
        int d = a.ids[(int64_t)b * G + jj];
        if (d != i) {
          n = jj;
          gn = i;
          decided = true;
        }
      }
    }
  }
  int32_t* out = a.out_tokens + (int64_t)b * G1;
  if (nan_any) {
    for (int jj = lane; jj < G1; jj += kWave) out[jj] = -1;
    if (lane == 0) {
      a.out_nacc[b] = 0;
      if (a.out_flags) a.out_flags[b] = 8u;
    }
    return;
  }
  for (int jj = lane; jj < G1; jj += kWave) out[jj] = jj < n ? a.ids[(int64_t)b * G + jj] : (jj == n ? gn : -1);
  if (lane == 0) {
    a.out_nacc[b] = n;
    uint32_t fl = 0;
    if (n < G) {
      int d = a.ids[(int64_t)b * G + n];
      if (d < 0 || (int64_t)d >= a.V) fl |= 1u;
    }
    if (a.out_flags) a.out_flags[b] = fl;
  }
}

// ---------------------------------------------------------------------------
// Statistics ([WR] §4.2, [RL] §2): per (row, chunk) partial sums, then a
// per-row finish.  Rows with a stored kept list need only sum(q) from the
// chunk pass; the min / positive-part sums over the kept set come from the
// list.  Other rows stream logits and q together.
// ---------------------------------------------------------------------------
struct StatsArgs {
  const void* logits;
  const float* q;
  const int32_t* ids;
  int64_t V;
  int32_t gamma;
  int32_t nchunks;
  int64_t chunk;
  float c;
  const RowInfo* info;  // [B * gamma]
  const Cand* kept;
  int32_t kmax;
  double* partials;     // [rows][nchunks][4]
  float* out_alpha;
  float* out_zpq;
  float* out_zqp;
  float* out_acc;
  int64_t rows;
};

template <bool BF16>
__global__ void __launch_bounds__(256) stats_chunk_kernel(StatsArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t blk = blockIdx.x;
  const int64_t r = blk / a.nchunks;
  const int ci = (int)(blk - r * a.nchunks);
  const RowInfo ri = a.info[r];
  const int b = (int)(r / a.gamma), j = (int)(r - (int64_t)b * a.gamma);
  const int64_t lrow = ((int64_t)b * (a.gamma + 1) + j) * a.V;
  const int64_t qrowo = r * a.V;
  const int64_t x0 = (int64_t)ci * a.chunk, x1 = min(x0 + a.chunk, a.V);
  double mn = 0.0, pq = 0.0, qp = 0.0, sq = 0.0;
  __shared__ double s_p[4][4];
  if (!(ri.flags & RF_NONFINITE)) {
    const bool big = (ri.flags & RF_BIG) != 0;
    const double invS = 1.0 / ri.S;
    for (int64_t x = x0 + tid; x < x1; x += 256) {
      double qv = (double)a.q[qrowo + x];
      if (big) {
        float z = load_logit<BF16>(a.logits, lrow + x);
        double p = (z >= ri.tau) ? (double)e_of(z, a.c, ri.R) * invS : 0.0;
        double d = p - qv;
        mn += fmin(p, qv);
        if (d > 0.0) pq += d;
        if (d < 0.0) qp -= d;
      } else {
        sq += qv;
      }
    }
  }
  mn = wave_sum_d(mn);
  pq = wave_sum_d(pq);
  qp = wave_sum_d(qp);
  sq = wave_sum_d(sq);
  if (lane == 0) {
    s_p[wid][0] = mn;
    s_p[wid][1] = pq;
    s_p[wid][2] = qp;
    s_p[wid][3] = sq;
  }
  __syncthreads();
  if (tid < 4) {
    double v = ((s_p[0][tid] + s_p[1][tid]) + s_p[2][tid]) + s_p[3][tid];
    a.partials[(r * a.nchunks + ci) * 4 + tid] = v;
  }
}

__global__ void __launch_bounds__(256) stats_final_kernel(StatsArgs a) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * 4 + wid;
  if (r >= a.rows) return;
  const RowInfo ri = a.info[r];
  const float qnan = __builtin_nanf("");
  if (ri.flags & RF_NONFINITE) {
    if (lane == 0) {
      a.out_alpha[r] = qnan;
      a.out_zpq[r] = qnan;
      a.out_zqp[r] = qnan;
      a.out_acc[r] = qnan;
    }
    return;
  }
  double acc4[4] = {0.0, 0.0, 0.0, 0.0};
  for (int k = 0; k < 4; ++k) {
    double v = 0.0;
    for (int c = lane; c < a.nchunks; c += kWave) v += a.partials[(r * a.nchunks + c) * 4 + k];
    acc4[k] = wave_sum_d(v);
  }
  const double invS = 1.0 / ri.S;
  double alpha, zpq, zqp;
  if (ri.flags & RF_BIG) {
    alpha = acc4[0];
    zpq = acc4[1];
    zqp = acc4[2];
  } else {
    const Cand* L = a.kept + r * a.kmax;
    const float* qr = a.q + r * a.V;
    double mn = 0.0, pq = 0.0, qp = 0.0, sqk = 0.0;
    for (int i = lane; i < ri.nkept; i += kWave) {
      Cand e = L[i];
      double p = (double)e.v * invS;
      double qv = (double)qr[e.idx];
      double d = p - qv;
      mn += fmin(p, qv);
      if (d > 0.0) pq += d;
      if (d < 0.0) qp -= d;
      sqk += qv;
    }
    mn = wave_sum_d(mn);
    pq = wave_sum_d(pq);
    qp = wave_sum_d(qp);
    sqk = wave_sum_d(sqk);
    alpha = mn;
    zpq = pq;
    zqp = (acc4[3] - sqk) + qp;
  }
  if (lane == 0) {
    a.out_alpha[r] = (float)alpha;
    a.out_zpq[r] = (float)zpq;
    a.out_zqp[r] = (float)zqp;
    float ap;
    if (ri.d < 0) ap = qnan;
    else if (ri.qd == 0.0f) ap = ri.ed > 0.0f ? 1.0f : 0.0f;
    else ap = (float)fmin(1.0, ((double)ri.ed * invS) / (double)ri.qd);
    a.out_acc[r] = ap;
  }
}

}  // namespace sv
