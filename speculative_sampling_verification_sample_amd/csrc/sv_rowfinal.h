// K2 -- per-row finalisation of the processed target distribution p, with
// the exact multi-pass path for rows the candidate lists cannot settle.
//
// One workgroup per row merges the chunk results: the row max gives the
// integral reference R, the chunk sums give the full-row mass S
// (temperature softmax, [WR] §7.2).  With truncation ([WR] §7.3) it builds
// the candidate union in LDS (every element >= the highest chunk threshold
// is in it) and selects by radix passes over order-preserving keys
//   top-k : keep every token whose logit >= the k-th largest logit;
//   top-p : keep the most probable tokens until their mass reaches
//           top_p * S (on the top-k set when both are active), plus ties
//           (masses as 2^40 fixed point, so sums are exact and order-free).
// The kept set is stored as a list of (logit, id) in token-id order (for the
// inverse CDF) together with S over it and S64, the double sum of its e64
// (the normaliser of the draws and the statistics).  It also reads this row's draft logit and q(d) so
// the acceptance test needs no further pass ([WR] §6).
#pragma once

#include <type_traits>

#include "sv_device.h"

namespace sv {

struct RowFinalArgs {
  const void* logits;
  QSrc q;               // draft distribution, one row per draft position
  const int32_t* ids;   // one id per draft position
  int64_t V;
  int32_t rows_per_req;
  int32_t G1;
  int32_t gamma;
  const int32_t* cu;    // ragged draft offsets [B + 1], or null
  int32_t n_live;       // ragged: packed rows that exist (n_draft + B)
  int32_t nchunks;
  int32_t cap_out;
  int32_t trunc;        // 0: untruncated rows, 1: top-k and/or top-p
  int32_t fast;         // 0: every truncated row takes the exact multi-pass path
  int32_t top_k;        // active when 0 < top_k < V
  float top_p;          // active when < 1
  float c;
  float c2, cl;         // two-part log2(e) / T (untruncated rows' e2)
  double c64;           // log2(e) / T (e64)
  int32_t um;           // LDS capacity (power of two) for the candidate union
  int32_t kmax;         // capacity of a stored kept list
  int32_t scale_bits;   // fixed-point bits of the exact path's mass histogram
  const ChunkOut* cout;
  const Cand* cand;
  RowInfo* info;        // [rows]
  Cand* kept;           // [rows][kmax]  (v = z(x), the logit; idx = token id), id order
};

// Draft gather for a row whose kept set and normaliser are final: the
// draft's logit, its float exponential and q(d) (the acceptance test needs
// them with S, or with S64).  dpos is the row's draft position, < 0 for a
// row without a draft (the bonus row).  (ch, cl): e2's two-part c on
// untruncated rows (their S sums e2), (c, 0) on truncated ones (S sums e).
template <bool BF16>
__device__ __forceinline__ void gather_draft_at(const void* logits, const QSrc& q, const int32_t* ids, int64_t V,
                                                float ch, float cl, int64_t dpos, int64_t rowoff, RowInfo& ri) {
  ri.ed = 0.0f;
  ri.qd = 0.0f;
  ri.d = -1;
  ri.zd = 0.0f;
  if (dpos < 0) return;
  int d = ids[dpos];
  if (d < 0 || (int64_t)d >= V) {
    ri.d = -2;
    return;
  }
  ri.d = d;
  float z = load_logit<BF16>(logits, rowoff + d);
  ri.zd = z;
  ri.ed = (z >= ri.tau) ? e2_of(z, ch, cl, ri.R) : 0.0f;
  ri.qd = q_at(q, dpos, d);
}

template <bool BF16>
__device__ __forceinline__ void gather_draft(const RowFinalArgs& a, int64_t dpos, int64_t rowoff, RowInfo& ri) {
  gather_draft_at<BF16>(a.logits, a.q, a.ids, a.V, a.trunc ? a.c : a.c2, a.trunc ? 0.0f : a.cl, dpos, rowoff, ri);
}


// Merge the chunk results of one row in chunk order (one thread).
struct RowMerge {
  float xmax, thr, R;
  uint32_t flags;
  double S;  // full-row mass against R (0 when the pass kept no sums)
};
__device__ inline RowMerge merge_chunks(const ChunkOut* co, int nchunks, float c) {
  RowMerge m;
  m.xmax = kNegInf;
  m.thr = kLowest;
  m.flags = 0;
  double s = 0.0;
  float Rs = kNegInf;
  for (int k0 = 0; k0 < nchunks; k0 += 8) {
    ChunkOut o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (k0 + i < nchunks) o[i] = co[k0 + i];  // loads issued together
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (k0 + i >= nchunks) break;
      m.xmax = fmaxf(m.xmax, o[i].xmax);
      m.thr = fmaxf(m.thr, o[i].thr);
      m.flags |= o[i].flags;
      sr_merge(s, Rs, o[i].s, o[i].Rs);
    }
  }
  m.R = ceilf(m.xmax * c);
  m.S = (Rs == kNegInf) ? 0.0 : ldexp(s, (int)(Rs - m.R));
  return m;
}
__device__ inline bool merge_nonfinite(const RowMerge& m) {
  // a NaN logit poisons the exp sums of the modes that keep them (S != S)
  return (m.flags & (CF_NAN | CF_POSINF)) || !(m.xmax > kNegInf) || !(fabsf(m.R) < kPosInf) || (m.S != m.S);
}

// Row info of an untruncated row straight from its chunk results; the
// draft's logit and q(d) come from the row pass's gather (gath[grow], the
// plan row) when `gath` is set.
template <bool BF16>
__device__ RowInfo untrunc_row_info(const ChunkOut* co, int nchunks, float c, float c2, float cl, const void* logits,
                                    const QSrc& q, const int32_t* ids, int64_t V, int64_t dpos, int64_t rowoff,
                                    const float2* gath = nullptr, int64_t grow = 0) {
  // the draft's id and gathered (z(d), q(d)) do not depend on the merge:
  // their loads go out first, with the chunk results'
  int dg = -1;
  float2 g = make_float2(0.0f, 0.0f);
  if (gath != nullptr && dpos >= 0) {
    dg = ids[dpos];
    g = gath[grow];
  }
  RowMerge m = merge_chunks(co, nchunks, c);
  RowInfo ri;
  ri.S = m.S;
  ri.S64 = 0.0;
  ri.R = m.R;
  ri.tau = kLowest;
  ri.nkept = -1;
  ri.flags = RF_BIG;
  ri.ed = 0.0f;
  ri.qd = 0.0f;
  ri.d = -1;
  ri.zd = 0.0f;
  if (merge_nonfinite(m)) {
    ri.flags = RF_NONFINITE;
    return ri;
  }
  if (gath != nullptr) {
    if (dpos >= 0) {
      const int d = dg;
      if (d < 0 || (int64_t)d >= V) {
        ri.d = -2;
      } else {
        ri.d = d;
        ri.zd = g.x;
        ri.ed = (g.x >= ri.tau) ? e2_of(g.x, c2, cl, ri.R) : 0.0f;
        ri.qd = g.y;
      }
    }
    return ri;
  }
  gather_draft_at<BF16>(logits, q, ids, V, c2, cl, dpos, rowoff, ri);
  return ri;
}

// ---- block-level selection over an LDS candidate array (256 threads) ----
// Fixed-point masses (e * 2^40, e <= ~1) make every sum an integer sum, so
// results do not depend on the order of the additions.
constexpr int kMassBits = 40;

__device__ __forceinline__ unsigned long long to_fixed(float e) {
  return (unsigned long long)rint((double)e * 1099511627776.0);  // 2^40
}

__device__ unsigned long long block_sum_u64(unsigned long long v, unsigned long long* s_tmp /*[4]*/) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
v = wave_sum_u64(v);
  __syncthreads();
  if (lane == 0) s_tmp[wid] = v;
  __syncthreads();
  unsigned long long t = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
  __syncthreads();
  return t;
}

// Key of the `need`-th largest entry of the list (counted with multiplicity).
template <bool BF16>
__device__ uint32_t block_select_count(const uint32_t* keys, int n, int need, uint32_t* hist, int* s_dn) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  constexpr int kLow = BF16 ? 16 : 0;
  uint32_t prefix = 0, pmask = 0;
  for (int shift = 24; shift >= kLow; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int i0 = 0; i0 < n; i0 += 256) {
      const int i = i0 + tid;
      const uint32_t k = i < n ? keys[i] : 0u;
      if (i < n && (k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wid == 0) {
      int d = wave_find_digit(hist, need);
      if (lane == 0) {
        s_dn[0] = d;
        s_dn[1] = need;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)s_dn[0] << shift;
    pmask |= 255u << shift;
    need = s_dn[1];
    __syncthreads();
  }
  return prefix;
}

// Largest key v with mass(entries with key >= v, key >= floor) >= target,
// an entry's mass being the fixed-point e(x) of its key (x = key2f(key)).
// Returns false when the whole mass stays below target.
template <bool BF16>
__device__ __forceinline__ bool block_select_mass(const uint32_t* keys, float c, float R, int n, uint32_t floor_key,
                                  double target, unsigned long long* mh, int* s_dn, unsigned long long* s_above,
                                  uint32_t& out_key) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  constexpr int kLow = BF16 ? 16 : 0;
  uint32_t prefix = 0, pmask = 0;
  if (tid == 0) *s_above = 0ull;
  for (int shift = 24; shift >= kLow; shift -= 8) {
    mh[tid] = 0ull;
    __syncthreads();
    for (int i0 = 0; i0 < n; i0 += 256) {
      const int i = i0 + tid;
      const uint32_t k = i < n ? keys[i] : 0u;
      if (i < n && k >= floor_key && (k & pmask) == prefix)
        atomicAdd(&mh[(k >> shift) & 255u], to_fixed(e_of(key2f(k), c, R)));
    }
    __syncthreads();
    if (wid == 0) {
      unsigned long long c0 = mh[255 - 4 * lane], c1 = mh[254 - 4 * lane], c2 = mh[253 - 4 * lane],
                         c3 = mh[252 - 4 * lane];
      const unsigned long long ls = c0 + c1 + c2 + c3, incl = wave_incl_scan_u64(ls);
      const unsigned long long above = *s_above;
      uint64_t hit = ballot((double)(above + incl) >= target);
      if (!hit) {
        if (lane == 0) s_dn[0] = -1;
      } else {
        const int src = (int)__builtin_ctzll(hit);
        if (lane == src) {
          unsigned long long run = above + (incl - ls);
          unsigned long long cs[4] = {c0, c1, c2, c3};
          int k = 0;
          for (; k < 3; ++k) {
            if ((double)(run + cs[k]) >= target) break;
            run += cs[k];
          }
          s_dn[0] = 255 - 4 * lane - k;
          *s_above = run;
        }
      }
    }
    __syncthreads();
    const int d = s_dn[0];
    __syncthreads();
    if (d < 0) return false;
    prefix |= (uint32_t)d << shift;
    pmask |= 255u << shift;
  }
  out_key = prefix;
  return true;
}

// Append entries to an LDS list with one atomic per wave (order arbitrary).
__device__ __forceinline__ int wave_append_slot(bool keep, int* counter) {
  const uint64_t m = ballot(keep);
  int base = 0;
  if (lane_id() == 0 && m) base = atomicAdd(counter, (int)__popcll(m));
  base = __shfl(base, 0, kWave);
  return base + lanes_below(m);
}

// ---------------------------------------------------------------------------
// Exact multi-pass path for rows the candidate lists cannot settle (run by
// the row finisher's workgroup): radix selection over the row in global
// memory.  top-k selects by count over order-preserving keys;
// top-p selects by mass with a fixed-point histogram (integer atomics, so the
// result does not depend on the order of the additions).
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ double block_sum_d(double v, double* s_tmp) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = wave_sum_d(v);
  __syncthreads();
  if (lane == 0) s_tmp[wid] = v;
  __syncthreads();
  double t = ((s_tmp[0] + s_tmp[1]) + (s_tmp[2] + s_tmp[3]));
  __syncthreads();
  return t;
}

template <bool BF16>
__device__ __forceinline__ void exact_row(const RowFinalArgs& a, int64_t r, int64_t dpos, int64_t rowoff, RowInfo ri,
                                          uint32_t* hist, unsigned long long* mhist) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t V = a.V;
  const float c = a.c;
  const float R = ri.R;

  // hist and mhist are the caller's selection histograms (LDS), free again
  // once every thread is here
  __syncthreads();
  __shared__ double s_tmp[4];
  __shared__ int s_digit, s_need, s_cnt[4];
  __shared__ unsigned long long s_above;
  constexpr int kLow = BF16 ? 16 : 0;
  // the lambdas below capture this copy, not the argument block, so that
  // the block is not copied to private memory and the loads stay global
  const void* const lg = a.logits;
  // tokens x .. x+7 of the row (-inf past V): one 16-byte load (two for
  // fp32) where the row is 16-byte aligned, else one load per token
  const bool rowvec = (rowoff % (BF16 ? 8 : 4)) == 0;
  auto seg8 = [&](int64_t x, float* z) {
    if (rowvec && x + 8 <= V) {
      if constexpr (BF16) {
        widen<true>(reinterpret_cast<const uint4*>(lg)[(rowoff + x) >> 3], z);
      } else {
        const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(lg) + rowoff + x);
        widen<false>(p[0], z);
        widen<false>(p[1], z + 4);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) z[e] = (x + e < V) ? load_logit<BF16>(lg, rowoff + x + e) : kNegInf;
    }
  };
  // body(x, z[8]) over the whole row in 8-token segments, lane-interleaved
  // (segment tid of every 256).  A lone workgroup is bound by load latency,
  // so batches of kEU segments per thread are loaded (as raw 16-byte words)
  // before any is used.
  constexpr int kW = BF16 ? 1 : 2;      // 16-byte words per segment
  constexpr int kEU = 2;                // segments in flight per thread
  auto load_whole = [&](int64_t x, uint4* w) {  // a whole aligned segment inside the row
    const uint4* p = BF16 ? reinterpret_cast<const uint4*>(lg) + ((rowoff + x) >> 3)
                          : reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(lg) + rowoff + x);
#pragma unroll
    for (int i = 0; i < kW; ++i) w[i] = p[i];
  };
  auto widen_seg = [&](const uint4* w, float* z) {
    if constexpr (BF16) {
      widen<true>(w[0], z);
    } else {
      widen<false>(w[0], z);
      widen<false>(w[1], z + 4);
    }
  };
  auto for_row = [&](auto&& body) {
    int64_t b0 = 0;
    if (rowvec) {
      for (; b0 + (int64_t)kEU * 2048 <= V; b0 += (int64_t)kEU * 2048) {
        uint4 ws[kEU][kW];
#pragma unroll
        for (int u = 0; u < kEU; ++u) load_whole(b0 + u * 2048 + tid * 8, ws[u]);
#pragma unroll
        for (int u = 0; u < kEU; ++u) {
          float zs[8];
          widen_seg(ws[u], zs);
          body(b0 + u * 2048 + tid * 8, zs);
        }
      }
    }
    for (int64_t x0 = b0 + (int64_t)tid * 8; x0 < V; x0 += 2048) {
      float zs[8];
      seg8(x0, zs);
      body(x0, zs);
    }
  };
  // the same over this thread's contiguous range [x0, x1) (x0 a multiple of 8)
  auto for_range = [&](int64_t x0, int64_t x1, auto&& body) {
    int64_t x = x0;
    if (rowvec) {
      for (; x + 8 * kEU <= x1; x += 8 * kEU) {
        uint4 ws[kEU][kW];
#pragma unroll
        for (int u = 0; u < kEU; ++u) load_whole(x + u * 8, ws[u]);
#pragma unroll
        for (int u = 0; u < kEU; ++u) {
          float zs[8];
          widen_seg(ws[u], zs);
          body(x + u * 8, zs);
        }
      }
    }
    for (; x < x1; x += 8) {
      float zs[8];
      seg8(x, zs);
      body(x, zs);
    }
  };

  // ---- top-k threshold (count) ----
  float tau = kLowest;
  const bool topk = a.top_k > 0 && (int64_t)a.top_k < V;
  if (topk) {
    uint32_t prefix = 0, pmask = 0;
    int need = a.top_k;
    int64_t nfinite = 0;
    for (int shift = 24; shift >= kLow; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      // per-thread runs of one bin are added with one atomic: a row's keys
      // share their upper bits, so the first passes land in few bins
      uint32_t cb = 0xffffffffu, ca = 0;
      for_row([&](int64_t, const float* zs) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (!(zs[e] > kNegInf)) continue;
          const uint32_t key = f2key(zs[e]);
          if ((key & pmask) == prefix) {
            const uint32_t bin = (key >> shift) & 255u;
            if (bin == cb) {
              ++ca;
            } else {
              if (ca) atomicAdd(&hist[cb], ca);
              cb = bin;
              ca = 1;
            }
          }
        }
      });
      if (ca) atomicAdd(&hist[cb], ca);
      __syncthreads();
      if (shift == 24) {
        int64_t tot = 0;
        for (int k = 0; k < 256; ++k) tot += hist[k];
        nfinite = tot;
        if (nfinite < need) break;
      }
      if (wid == 0) {
        int d = wave_find_digit(hist, need);
        if (lane == 0) {
          s_digit = d;
          s_need = need;
        }
      }
      __syncthreads();
      prefix |= (uint32_t)s_digit << shift;
      pmask |= 255u << shift;
      need = s_need;
      __syncthreads();
    }
    if (nfinite >= a.top_k) tau = key2f(prefix);
  }
  // ---- top-p threshold (mass), against the mass of the top-k set (without
  //      top-k: the row's mass from the chunk sums, as on the fast path) ----
  if (a.top_p < 1.0f) {
    double Sk = ri.S;
    if (topk) {
      double part = 0.0;
      for_row([&](int64_t, const float* zs) {
        float f = 0.0f;  // a segment's 8 terms (each <= 1) in float, then into the double
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (zs[e] >= tau) f += e_of(zs[e], c, R);
        part += (double)f;
      });
      Sk = block_sum_d<BF16>(part, s_tmp);
    }
    const double sc = ldexp(1.0, a.scale_bits);
    const double target = (double)a.top_p * Sk * sc;
    uint32_t prefix = 0, pmask = 0;
    if (tid == 0) s_above = 0ull;
    bool found_all = true;
    for (int shift = 24; shift >= kLow; shift -= 8) {
      mhist[tid] = 0ull;
      __syncthreads();
      uint32_t cb = 0xffffffffu;
      unsigned long long ca = 0ull;
      for_row([&](int64_t, const float* zs) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (!(zs[e] >= tau)) continue;
          const uint32_t key = f2key(zs[e]);
          if ((key & pmask) == prefix) {
            const uint32_t bin = (key >> shift) & 255u;
            const unsigned long long m = (unsigned long long)rint((double)e_of(zs[e], c, R) * sc);
            if (bin == cb) {
              ca += m;
            } else {
              if (cb != 0xffffffffu) atomicAdd(&mhist[cb], ca);
              cb = bin;
              ca = m;
            }
          }
        }
      });
      if (cb != 0xffffffffu) atomicAdd(&mhist[cb], ca);
      __syncthreads();
      if (wid == 0) {
        // lane l holds bins 255-4l .. 252-4l
        unsigned long long c0 = mhist[255 - 4 * lane], c1 = mhist[254 - 4 * lane], c2 = mhist[253 - 4 * lane],
                           c3 = mhist[252 - 4 * lane];
        unsigned long long ls = c0 + c1 + c2 + c3;
        const unsigned long long incl = wave_incl_scan_u64(ls);
        unsigned long long above = s_above;
        uint64_t hit = ballot((double)(above + incl) >= target);
        int src = hit ? (int)__builtin_ctzll(hit) : -1;
        if (src < 0) {
          if (lane == 0) s_digit = -1;
        } else if (lane == src) {
          unsigned long long run = above + (incl - ls);
          unsigned long long cs[4] = {c0, c1, c2, c3};
          int k = 0;
          for (; k < 3; ++k) {
            if ((double)(run + cs[k]) >= target) break;
            run += cs[k];
          }
          s_digit = 255 - 4 * lane - k;
          s_above = run;
        }
      }
      __syncthreads();
      int d = s_digit;
      __syncthreads();
      if (d < 0) {
        found_all = false;
        break;
      }
      prefix |= (uint32_t)d << shift;
      pmask |= 255u << shift;
    }
    if (found_all) tau = fmaxf(tau, key2f(prefix));
  }
  // ---- the kept set {z >= tau}: each thread takes one contiguous segment
  //      of the row (segments in id order), counts and weighs its kept
  //      tokens, and after one block scan writes them at their place in the
  //      id-ordered list (no barrier inside the passes over the row) ----
  const int64_t seglen = ((V + 255) / 256 + 7) / 8 * 8;
  const int64_t sx0 = min((int64_t)tid * seglen, V), sx1 = min(sx0 + seglen, V);
  int cntp = 0;
  double part = 0.0;
  for_range(sx0, sx1, [&](int64_t, const float* zs) {
    float f = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (zs[e] >= tau) {
        ++cntp;
        f += e_of(zs[e], c, R);
      }
    }
    part += (double)f;
  });
  // S64 in a pass of its own, one token at a time (its double exponentials
  // would otherwise raise the register count of the whole row finisher)
  double part64 = 0.0;
  if (cntp > 0) {
    const double c64 = a.c64;
    for (int64_t x = sx0; x < sx1; ++x) {
      const float zx = load_logit<BF16>(lg, rowoff + x);
      if (zx >= tau) part64 += e64_of(zx, c64, R);
    }
  }
  // fixed segments and order: deterministic
  const double S = block_sum_d<BF16>(part, s_tmp);
  const double S64 = block_sum_d<BF16>(part64, s_tmp);
  const int incl = wave_incl_scan_i(cntp);
  if (lane == kWave - 1) s_cnt[wid] = incl;
  __syncthreads();
  int before = incl - cntp;
  for (int w = 0; w < wid; ++w) before += s_cnt[w];
  const int nkept = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
  __syncthreads();
  ri.tau = tau;
  ri.S = S;
  ri.S64 = S64;
  ri.flags = 0;
  if (nkept > a.kmax) {
    ri.flags = RF_BIG;
    ri.nkept = -1;
  } else {
    Cand* out = a.kept + r * (int64_t)a.kmax;
    int pos = before;
    if (cntp > 0) {
      for_range(sx0, sx1, [&](int64_t x, const float* zs) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (zs[e] >= tau) {
            Cand ce;
            ce.idx = (int32_t)(x + e);
            ce.v = zs[e];
            out[pos++] = ce;
          }
        }
      });
    }
    ri.nkept = nkept;
  }
  if (tid == 0) {
    gather_draft<BF16>(a, dpos, rowoff, ri);
    a.info[r] = ri;
  }
}

template <bool BF16>
__global__ void __launch_bounds__(256, BF16 ? 6 : 1) rowfinal_kernel(RowFinalArgs a) {
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  const RowAt at = row_at(a.cu, a.n_live, a.rows_per_req, a.G1, a.gamma, a.V, r);
  if (!at.live) return;  // past the rows of a ragged batch
  const int64_t rowoff = at.rowoff, dpos = at.dpos;

  __shared__ float s_xm, s_th, s_R;
  __shared__ double s_S;
  __shared__ uint32_t s_fl;
  __shared__ int s_n, s_dn[2];
  __shared__ int s_nc[kWave], s_maxnc;  // candidates per chunk (<= 64 chunks)
  __shared__ int s_gd;                 // draft gather, read early by one lane of wave 1
  __shared__ float s_gz, s_gq;
  __shared__ uint32_t hist[256];
  __shared__ unsigned long long mh[256], s_u64[4], s_above;
  extern __shared__ __align__(16) unsigned char s_dyn[];
  // union entries: keys and token ids (an entry's fixed-point mass is a
  // function of its key, recomputed where needed, which halves the LDS a
  // workgroup holds and so doubles the row finishers resident per CU)
  uint32_t* keys = reinterpret_cast<uint32_t*>(s_dyn);
  int32_t* idxs = reinterpret_cast<int32_t*>(s_dyn + (size_t)a.um * 4);

  const int nch = a.nchunks;
  const bool flat = nch <= kWave;  // the union walks one flat index over the chunk lists
  // The draft's id, logit and q(d) are fetched by lane 0 of wave 1 while
  // wave 0 merges the chunks, so the row's result does not wait on them.
  const bool has_draft = dpos >= 0;
  int gd = -1;
  float gz = 0.0f, gq = 0.0f;
  if (tid == kWave && has_draft) gd = a.ids[dpos];
  // Candidate loads are issued now, before the chunk counts are known:
  // thread t takes slots t / nch + u * per of chunk t % nch (per = 256 / nch),
  // every slot inside the list's capacity; the counts decide later which
  // loads hold candidates.
  constexpr int kU = 4;
  const Cand* cd = a.cand + r * nch * (int64_t)a.cap_out;
  const int per = flat ? 256 / nch : 0;
  const int cmine = flat ? tid % nch : 0;
  const int s0 = flat ? tid / nch : 0;
  Cand pre[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    pre[u].v = kNegInf;
    pre[u].idx = 0;
    const int sl = s0 + u * per;
    if (a.trunc && flat && tid < per * nch && sl < a.cap_out) pre[u] = cd[(int64_t)cmine * a.cap_out + sl];
  }
  if (tid < kWave) {
    // wave 0 merges the chunk results (lane l: chunks l, l + 64, ...)
    const int lane = tid;
    const ChunkOut* co = a.cout + r * nch;
    float xm = kNegInf, th = kLowest, Rs = kNegInf;
    uint32_t flg = 0;
    double ss = 0.0;
    int ncl = 0;
    for (int c = lane; c < nch; c += kWave) {
      const ChunkOut o = co[c];
      xm = fmaxf(xm, o.xmax);
      th = fmaxf(th, o.thr);
      flg |= o.flags;
      sr_merge(ss, Rs, o.s, o.Rs);
      ncl = o.ncand;
    }
    xm = wave_max(xm);
    th = wave_max(th);
    flg = wave_or(flg);
    const float Rm = wave_max(Rs);
    double sl = 0.0;
    if (Rs != kNegInf) sl = ldexp(ss, (int)(Rs - Rm));
    ss = wave_sum_d(sl);
    if (flat) {
      s_nc[lane] = ncl;
      const int mx = (int)wave_max_u32((uint32_t)ncl);
      if (lane == 0) s_maxnc = mx;
    }
    if (lane == 0) {
      const float Rrow = ceilf(xm * a.c);
      s_xm = xm;
      s_th = th;
      s_fl = flg;
      s_R = Rrow;
      s_S = (Rm == kNegInf) ? 0.0 : ldexp(ss, (int)(Rm - Rrow));
      s_n = 0;
    }
  }
  __syncthreads();
  RowInfo ri;
  ri.S = s_S;
  ri.S64 = 0.0;
  ri.R = s_R;
  ri.tau = kLowest;
  ri.nkept = -1;
  ri.flags = 0;
  ri.ed = 0.0f;
  ri.qd = 0.0f;
  ri.d = -1;
  ri.zd = 0.0f;
  const uint32_t fl = s_fl;
  if ((fl & (CF_NAN | CF_POSINF)) || !(s_xm > kNegInf) || !(fabsf(s_R) < kPosInf) || (s_S != s_S)) {
    if (tid == 0) {
      ri.flags = RF_NONFINITE;
      a.info[r] = ri;
    }
    return;
  }
  if (!a.trunc) {
    if (tid == 0) {
      ri.flags = RF_BIG;
      gather_draft<BF16>(a, dpos, rowoff, ri);
      a.info[r] = ri;
    }
    return;
  }
  if ((fl & CF_OVERFLOW) || !a.fast) {
    exact_row<BF16>(a, r, dpos, rowoff, ri, hist, mh);
    return;
  }

  if (tid == kWave && gd >= 0 && (int64_t)gd < a.V) {
    gz = load_logit<BF16>(a.logits, rowoff + gd);
    gq = q_at(a.q, dpos, gd);
  }

  // ---- candidate union (entries >= the highest chunk threshold) ----
  const float theta = s_th;
  const float R = s_R;
  auto add_union = [&](bool valid, const Cand& e) {
    const bool keep = valid && e.v >= theta;
    const int pos = wave_append_slot(keep, &s_n);
    if (keep && pos < a.um) {
      keys[pos] = f2key(e.v);
      idxs[pos] = e.idx;
    }
  };
  if (flat) {
    const bool mine = tid < per * nch;
    const int ncm = mine ? s_nc[cmine] : 0;
#pragma unroll
    for (int u = 0; u < kU; ++u) add_union(mine && s0 + u * per < ncm, pre[u]);
    // lists longer than kU * per entries (uniform trip count)
    for (int sl0 = kU * per; sl0 < s_maxnc; sl0 += per) {
      const int sl = sl0 + s0;
      const bool v = mine && sl < ncm;
      Cand e;
      e.v = kNegInf;
      e.idx = 0;
      if (v) e = cd[(int64_t)cmine * a.cap_out + sl];
      add_union(v, e);
    }
  } else {
    for (int c = 0; c < nch; ++c) {
      const int nc = a.cout[r * nch + c].ncand;
      for (int i0 = 0; i0 < nc; i0 += 256) {
        const int i = i0 + tid;
        Cand e;
        e.v = kNegInf;
        e.idx = 0;
        if (i < nc) e = cd[(int64_t)c * a.cap_out + i];
        add_union(i < nc, e);
      }
    }
  }
  if (tid == kWave) {
    s_gd = gd;
    s_gz = gz;
    s_gq = gq;
  }
  __syncthreads();
  const int nu = s_n;
  if (nu > a.um) {
    exact_row<BF16>(a, r, dpos, rowoff, ri, hist, mh);
    return;
  }

  // ---- thresholds ----
  const bool topk = a.top_k > 0 && (int64_t)a.top_k < a.V;
  const bool topp = a.top_p < 1.0f;
  uint32_t kfloor = 0;  // keys below this are outside the top-k set
  if (topk && nu >= a.top_k) kfloor = block_select_count<BF16>(keys, nu, a.top_k, hist, s_dn);
  auto mass_from = [&](uint32_t kf) -> unsigned long long {
    unsigned long long part = 0ull;
    for (int i = tid; i < nu; i += 256)
      if (keys[i] >= kf) part += to_fixed(e_of(key2f(keys[i]), a.c, R));
    return block_sum_u64(part, s_u64);
  };
  uint32_t kfinal = kfloor;
  const double scale = 1099511627776.0;  // 2^40
  if (topp) {
    const double Sref = topk ? (double)mass_from(kfloor) : s_S * scale;
    const double target = (double)a.top_p * Sref;
    uint32_t kp;
    if (block_select_mass<BF16>(keys, a.c, R, nu, kfloor, target, mh, s_dn, &s_above, kp)) {
      kfinal = kp;
    } else if (!(topk || theta == kLowest)) {
      // the crossing lies below the certified candidates: exact path
      exact_row<BF16>(a, r, dpos, rowoff, ri, hist, mh);
      return;
    }  // else rounding: keep the whole base set
  }
  const unsigned long long Sfx = mass_from(kfinal);
  ri.S = (double)Sfx / scale;
  ri.tau = key2f(kfinal);
  if (kfinal == 0) ri.tau = kLowest;
  // ---- kept list in token-id order: compact the kept entries (in any
  //      order) in place over the union (ids over the keys, logits over
  //      the ids), then store each at its rank by id (ids are unique within
  //      a row).  Each block of 256 entries is read before any of its slots
  //      is written; earlier blocks only write slots below the current one.
  //      S64 sums the entries' e64 as 2^53 fixed point, in 32-bit halves
  //      (the union holds at most 2048 entries, each e64 < 2, so neither
  //      half can overflow): integer sums, so S64 does not depend on the
  //      order of the additions, and a term of at least 1/2 (the row's
  //      largest is one) is taken exactly, so a kept set of one token has
  //      S64 = its e64 and p = 1 exactly, as in the plain definition. ----
  if (tid == 0) s_n = 0;
  __syncthreads();
  int32_t* kid = reinterpret_cast<int32_t*>(keys);
  float* kev = reinterpret_cast<float*>(idxs);
  for (int i0 = 0; i0 < nu; i0 += 256) {
    const int i = i0 + tid;
    const uint32_t k = i < nu ? keys[i] : 0u;
    const int id = i < nu ? idxs[i] : 0;
    const bool keep = i < nu && k >= kfinal;
    __syncthreads();
    const int pos = wave_append_slot(keep, &s_n);
    if (keep) {
      kid[pos] = id;
      kev[pos] = key2f(k);
    }
  }
  __syncthreads();
  const int nkept = s_n;
  unsigned long long s64hi = 0ull, s64lo = 0ull;
  for (int i = tid; i < nkept; i += 256) {
    const unsigned long long v = (unsigned long long)rint(e64_of(kev[i], a.c64, R) * 9007199254740992.0);  // 2^53
    s64hi += v >> 32;
    s64lo += v & 0xffffffffull;
  }
  s64hi = block_sum_u64(s64hi, s_u64);
  s64lo = block_sum_u64(s64lo, s_u64);
  const double S64 = ((double)s64hi * 4294967296.0 + (double)s64lo) * (1.0 / 9007199254740992.0);
  if (nkept <= a.kmax) {
    Cand* out = a.kept + r * (int64_t)a.kmax;
    // kid sits at the start of the dynamic LDS (16-byte aligned): ids are
    // read four at a time, the same address for every lane (a broadcast read).
    const int4* kid4 = reinterpret_cast<const int4*>(kid);
    const int nk4 = nkept >> 2;
    // KP entries ranked per thread in one sweep of 256 * KP entries
    auto sweep = [&](int i0, auto kp_tag) {
      constexpr int KP = decltype(kp_tag)::value;
      if (i0 + (tid & ~(kWave - 1)) >= nkept) return;  // this wave holds no entry
      int id[KP], rank[KP];
#pragma unroll
      for (int q = 0; q < KP; ++q) {
        const int i = i0 + q * 256 + tid;
        id[q] = i < nkept ? kid[i] : 0x7fffffff;
        rank[q] = 0;
      }
#pragma unroll 4
      for (int x = 0; x < nk4; ++x) {
        const int4 v = kid4[x];
#pragma unroll
        for (int q = 0; q < KP; ++q)
          rank[q] += (v.x < id[q] ? 1 : 0) + (v.y < id[q] ? 1 : 0) + (v.z < id[q] ? 1 : 0) + (v.w < id[q] ? 1 : 0);
      }
      for (int x = nk4 * 4; x < nkept; ++x) {
        const int v = kid[x];
#pragma unroll
        for (int q = 0; q < KP; ++q) rank[q] += v < id[q] ? 1 : 0;
      }
#pragma unroll
      for (int q = 0; q < KP; ++q) {
        const int i = i0 + q * 256 + tid;
        if (i < nkept) {
          Cand e;
          e.idx = id[q];
          e.v = kev[i];
          out[rank[q]] = e;
        }
      }
    };
    if (nkept <= 256) {
      sweep(0, std::integral_constant<int, 1>{});
    } else {
      for (int i0 = 0; i0 < nkept; i0 += 256 * 4) sweep(i0, std::integral_constant<int, 4>{});
    }
  }
  if (tid == 0) {
    if (nkept > a.kmax) {
      ri.flags = RF_BIG;
      ri.nkept = -1;
    } else {
      ri.nkept = nkept;
    }
    ri.ed = 0.0f;
    ri.qd = 0.0f;
    ri.d = -1;
    if (has_draft) {
      const int d = s_gd;
      if (d < 0 || (int64_t)d >= a.V) {
        ri.d = -2;
      } else {
        ri.d = d;
        ri.zd = s_gz;
        ri.ed = (s_gz >= ri.tau) ? e_of(s_gz, a.c, ri.R) : 0.0f;
        ri.qd = s_gq;
      }
    }
    ri.S64 = S64;
    a.info[r] = ri;
  }
}

}  // namespace sv
