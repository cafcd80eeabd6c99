// K1 -- the streaming pass over the logits (the HBM-bound hot loop).
//
// Every workgroup reads one chunk of one logits row with 16-byte loads
// (8 bf16 or 4 fp32 per load, 64 consecutive loads per wave) and writes a
// ChunkOut.  The grid is linear, nchunks * rows, chunk index fastest.
//
// rowpass_kernel, untruncated rows:
//   M_SOFTMAX : max and s = sum exp2(x*c - R)   (temperature softmax, [WR] §7.2)
//   M_ARGMAX  : max and the first index holding it    (greedy, [WR] §7.1)
//
// trunc_pass_kernel, rows under top-k / top-p ([WR] §7.3): max, optional s
// (top-p needs the full-row mass) and a candidate list holding every chunk
// element >= a threshold t0 that at least `nw` chunk elements reach.  Each
// thread keeps the max of every unit it streams, so t0 is chosen after the
// whole chunk is seen, and only the few units that reach it are read again:
//   - each thread's maximum over its units is one element of the chunk;
//   - each wave takes the ceil(nw/8)-th largest of its 64 thread maxima
//     (distinct threads hold distinct elements, so that many elements of
//     the wave reach it);
//   - t0 is the lowest of the 8 wave values, which therefore at least
//     8*ceil(nw/8) >= nw chunk elements reach.
// Any chunk's nw-th largest is <= the row's nw-th largest, so the merged
// lists contain every token of the row's top-k set (nw = k), and for top-p
// the row finisher certifies that the mass above the highest chunk
// threshold covers the nucleus.  A list longer than cap_out (ties, flat
// rows) is flagged CF_OVERFLOW and the row takes the exact path.
#pragma once

#include <type_traits>

#include "sv_device.h"

namespace sv {

enum { M_SOFTMAX = 0, M_ARGMAX = 1, M_TRUNC = 2 };

struct RowPassArgs {
  const void* logits;  // [B, G1, V]
  int64_t V;
  int64_t chunk;       // elements per chunk (multiple of 8)
  int32_t rows_per_req;
  int32_t G1;
  int32_t nchunks;
  float c;
  float c2, cl;        // two-part log2(e) / T (untruncated rows' e2 sums)
  int32_t nw;          // chunk elements the candidate threshold must certify
  int32_t cap_out;     // capacity of one chunk's list
  ChunkOut* out;  // [rows][nchunks]
  Cand* cand;     // [rows][nchunks][cap_out]
  // Optional draft gather (untruncated sampling): the workgroup whose chunk
  // holds d_j stores (z(d_j), q_j(d_j)) in gath[row].
  const int32_t* ids;
  QSrc q;
  int32_t gamma;
  float2* gath;
  // Ragged batches: draft offsets [B + 1] (null: uniform) and the packed
  // rows that exist (n_draft + B); workgroups past them return at once.
  const int32_t* cu;
  int32_t n_live;
};

constexpr int kTruncBS = 512;  // threads of the truncated-row pass

// Geometry of the chunk a workgroup owns: flat element range [F0, F1) and
// 16-byte unit range [U0, U1) (a unit may straddle the range ends).
struct ChunkGeom {
  int r, ci;
  bool live;
  int64_t dpos, rowoff, e0, e1, F0, F1, U0, U1;
};

template <int EPV>
__device__ __forceinline__ ChunkGeom chunk_geom(const RowPassArgs& a) {
  ChunkGeom g;
  const int64_t blk = blockIdx.x;
  g.r = (int)(blk / a.nchunks);
  g.ci = (int)(blk - (int64_t)g.r * a.nchunks);
  const RowAt at = row_at(a.cu, a.n_live, a.rows_per_req, a.G1, a.gamma, a.V, g.r);
  g.live = at.live;
  g.dpos = at.dpos;
  g.rowoff = at.rowoff;
  g.e0 = (int64_t)g.ci * a.chunk;
  g.e1 = min(g.e0 + a.chunk, a.V);
  g.F0 = g.rowoff + g.e0;
  g.F1 = g.rowoff + g.e1;
  g.U0 = g.F0 / EPV;
  g.U1 = (g.F1 + EPV - 1) / EPV;
  return g;
}

// Per-thread running statistics of the units it has seen: max, the online
// exponential sum (s, R) and NaN evidence.  The integral reference R lags
// the running max: it moves up (to ceil(max * c)) only when a unit's max
// times c passes R + kRefLag, so the exponentials stay within about
// 2^kRefLag and a wave seldom takes the rescale branch once its first
// units are in.  The row merges rescale every (s, R) to R = ceil(row max
// * c) exactly.  Unit
// sums collect in a float partial `sb` (at most 64 elements between
// flushes) that is folded into the double `s` by flush() and before every
// rescale.  The unit max ignores nothing: a NaN element makes it NaN, so
// such a unit never counts as a maximum (its row is flagged non-finite).
// TRACK_MAX = false: the caller keeps the running max itself (and stores it
// in xmax before finish_flags()).
constexpr float kRefLag = 16.0f;

// TWO_PART: the sums take e2 (the two-part c, cl set by the caller), else e.
template <bool BF16, bool DO_S, bool TRACK_MAX = true, bool TWO_PART = false>
struct UnitAcc {
  static constexpr int EPV = BF16 ? 8 : 4;
  float xmax = kNegInf;
  double s = 0.0;
  float sb = 0.0f;
  // Reference the exponentials use: the integral reference R once it
  // exists, before that a huge finite value, so finite logits add exactly 0
  // while NaN still reaches s (and +Inf, which the row flags anyway, makes
  // s infinite).
  float Re = 0x1p126f;
  // A unit max above vt moves R: (R + kRefLag) / c once R exists, -inf
  // before (so vt == -inf tells that there is no reference yet).
  float vt = kNegInf;
  uint32_t nan_words = 0;  // max of |bits| over whole units (per 16-bit half for bf16)
  uint32_t flags = 0;
  float c2 = 0.0f, cl = 0.0f;  // the two-part c (TWO_PART)

  // Widens a unit into x and returns its max.  rel is the chunk-relative
  // index of the unit's first element; with EDGE, elements outside [0, n)
  // become -inf.
  template <bool EDGE>
  __device__ __forceinline__ float add(const uint4& w, int rel, int n, float c, float (&x)[EPV]) {
    widen<BF16>(w, x);
    if constexpr (EDGE) {
#pragma unroll
      for (int i = 0; i < EPV; ++i) {
        if ((unsigned)(rel + i) >= (unsigned)n) x[i] = kNegInf;
        else if (x[i] != x[i]) flags |= CF_NAN;
      }
    } else if constexpr (!DO_S) {
      // no exp sums in this mode: NaN needs its own test (|bits| above +Inf)
      if constexpr (BF16) {
        const uint32_t m0 = w.x & 0x7fff7fffu, m1 = w.y & 0x7fff7fffu, m2 = w.z & 0x7fff7fffu, m3 = w.w & 0x7fff7fffu;
        const uint32_t lo = max(max(m0 & 0xffffu, m1 & 0xffffu), max(m2 & 0xffffu, m3 & 0xffffu));
        const uint32_t hi = max(max(m0 >> 16, m1 >> 16), max(m2 >> 16, m3 >> 16));
        nan_words = max(nan_words, max(lo, hi));
      } else {
        const uint32_t m = max(max(w.x & 0x7fffffffu, w.y & 0x7fffffffu), max(w.z & 0x7fffffffu, w.w & 0x7fffffffu));
        nan_words = max(nan_words, m);
      }
    }
    // NaN-propagating max (one v_maximum3_f32 per three elements)
    float vm = x[0];
#pragma unroll
    for (int i = 1; i < EPV; ++i) vm = __builtin_elementwise_maximum(vm, x[i]);
    if constexpr (TRACK_MAX) xmax = __builtin_elementwise_maximum(xmax, vm);
    if constexpr (DO_S) {
      if (vm > vt) {
        if (vm < kPosInf) {  // +Inf gets no reference (the row is flagged)
          const float Rn = ceilf(vm * c);
          s += (double)sb;
          if (vt != kNegInf) s = ldexp(s, (int)(Re - Rn));
          sb = 0.0f;
          Re = Rn;
          vt = (Rn + kRefLag) / c;
        }
      }
      // a NaN logit turns s into NaN, which the row merge reports
      float ev[EPV];
#pragma unroll
      for (int i = 0; i < EPV; ++i) {
        if constexpr (TWO_PART) ev[i] = e2_of(x[i], c2, cl, Re);
        else ev[i] = e_of(x[i], c, Re);
      }
      float t;
      if constexpr (EPV == 8) t = ((ev[0] + ev[1]) + (ev[2] + ev[3])) + ((ev[4] + ev[5]) + (ev[6] + ev[7]));
      else t = (ev[0] + ev[1]) + (ev[2] + ev[3]);
      sb += t;
    }
    return vm;
  }

  // The integral reference R of (s, R); -inf until a finite value is seen.
  __device__ __forceinline__ float ref() const { return vt == kNegInf ? kNegInf : Re; }

  __device__ __forceinline__ void flush() {
    if constexpr (DO_S) {
      s += (double)sb;
      sb = 0.0f;
    }
  }

  // After the last flush().
  __device__ __forceinline__ void finish_flags() {
    // merges drop sums without a reference: keep the evidence they carry
    // (only NaN or +Inf logits make such a sum nonzero)
    if constexpr (DO_S) {
      if (vt == kNegInf && s != 0.0) flags |= CF_NAN;
    }
    if constexpr (BF16) {
      if (nan_words > 0x7f80u) flags |= CF_NAN;
    } else {
      if (nan_words > 0x7f800000u) flags |= CF_NAN;
    }
    if (xmax == kPosInf) flags |= CF_POSINF;
  }
};

// Wave-wide merge of the (s, R) pairs: every lane's s is moved to the
// wave's largest reference by an exact power-of-two scaling, then summed in
// a fixed order (the wave reduction).
__device__ __forceinline__ void wave_sr_merge(double& s, float& R) {
  const float Rm = wave_max(R);
  double sl = 0.0;
  if (R != kNegInf) sl = ldexp(s, (int)(R - Rm));
  s = wave_sum_d(sl);
  R = Rm;
}

// ALIGNED: as for the truncated pass, the host has checked that every unit
// in range is whole, so the edge variant of the unit code is left out.
template <int MODE, bool BF16, int BS, bool ALIGNED>
__global__ void __launch_bounds__(BS) rowpass_kernel(RowPassArgs a) {
  constexpr int EPV = BF16 ? 8 : 4;
  constexpr int NWV = BS / kWave;
  constexpr bool DO_S = (MODE == M_SOFTMAX);

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const ChunkGeom g = chunk_geom<EPV>(a);
  const uint4* __restrict__ base = reinterpret_cast<const uint4*>(a.logits);
  const float c = a.c;

  __shared__ float s_xm[NWV];
  __shared__ int s_ai[NWV];
  __shared__ double s_s[NWV];
  __shared__ float s_R[NWV];
  __shared__ uint32_t s_fl[NWV];

  if (!g.live) return;
  if (a.gath != nullptr && tid == 0 && g.dpos >= 0) {
    const int d = a.ids[g.dpos];
    if ((int64_t)d >= g.e0 && (int64_t)d < g.e1) {
      const float zd = BF16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(a.logits)[g.rowoff + d] << 16)
                            : reinterpret_cast<const float*>(a.logits)[g.rowoff + d];
      a.gath[g.r] = make_float2(zd, q_at(a.q, g.dpos, d));
    }
  }

  // untruncated sums take the two-part c: the acceptance test compares
  // against them directly
  UnitAcc<BF16, DO_S, MODE != M_ARGMAX, true> acc;
  acc.c2 = a.c2;
  acc.cl = a.cl;
  float bestv = kNegInf;  // running max (argmax mode)
  int aidx = 0x7fffffff;  // row index of this thread's first maximum

  auto process = [&](int64_t u, const uint4& w, auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    float x[EPV];
    const float vm = acc.template add<EDGE>(w, (int)(u * EPV - g.F0), (int)(g.F1 - g.F0), c, x);
    if constexpr (MODE == M_ARGMAX) {
      // units arrive in increasing order, so a strictly larger max is the
      // only case that moves the first maximum; rare after the first units
      if (vm > bestv) {
        bestv = vm;
        int first = 0;
#pragma unroll
        for (int i = EPV - 1; i >= 0; --i)
          if (x[i] == vm) first = i;
        aidx = (int)(u * EPV + first - g.rowoff);
      }
    }
  };

  using Edge = std::true_type;
  using NoEdge = std::false_type;

  // Step k gives thread tid the unit U0 + k*BS + tid; up to kUnroll units'
  // loads are issued before any is processed.
  constexpr int kUnroll = 8;
  const bool aligned = ALIGNED || ((g.F0 % EPV == 0) && (g.F1 % EPV == 0));
  const int64_t nunits = g.U1 - g.U0;
  const int64_t nsteps = (nunits + BS - 1) / BS;
  const int64_t nfull = aligned ? nunits / BS : 0;  // steps whose units are all whole and in range
  for (int64_t k0 = 0; k0 < nsteps; k0 += kUnroll) {
    uint4 wv[kUnroll];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      const int64_t u = g.U0 + (k0 + i) * BS + tid;
      wv[i] = make_uint4(0u, 0u, 0u, 0u);
      if (k0 + i < nsteps && u < g.U1) wv[i] = ld_stream(base + u);
    }
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      if (k0 + i >= nsteps) break;
      const int64_t u = g.U0 + (k0 + i) * BS + tid;
      if constexpr (ALIGNED) {
        if (k0 + i < nfull || u < g.U1) process(u, wv[i], NoEdge{});
      } else if (k0 + i < nfull) {
        process(u, wv[i], NoEdge{});
      } else if (u < g.U1) {
        process(u, wv[i], Edge{});
      }
    }
    acc.flush();
  }
  if constexpr (MODE == M_ARGMAX) acc.xmax = bestv;
  acc.finish_flags();

  // ---- workgroup reductions (fixed order) ----
  float wxm = acc.xmax;
  int wai = aidx;
  if constexpr (MODE == M_ARGMAX) wave_argmax(wxm, wai);
  else wxm = wave_max(wxm);
  const uint32_t wfl = wave_or(acc.flags);
  double ws = acc.s;
  float wR = acc.ref();
  if constexpr (DO_S) wave_sr_merge(ws, wR);
  if (lane == 0) {
    s_xm[wid] = wxm;
    s_ai[wid] = wai;
    s_s[wid] = ws;
    s_R[wid] = wR;
    s_fl[wid] = wfl;
  }
  __syncthreads();
  if (wid == 0) {
    // wave 0 merges the per-wave partials (lane l holds wave l's)
    const bool own = lane < NWV;
    float xm = own ? s_xm[lane] : kNegInf;
    int ai = own ? s_ai[lane] : 0x7fffffff;
    uint32_t fl = own ? s_fl[lane] : 0u;
    double ss = own ? s_s[lane] : 0.0;
    float RR = own ? s_R[lane] : kNegInf;
    if constexpr (MODE == M_ARGMAX) wave_argmax(xm, ai);
    else xm = wave_max(xm);
    fl = wave_or(fl);
    if constexpr (DO_S) wave_sr_merge(ss, RR);
    if (MODE == M_ARGMAX && xm == kNegInf) ai = (int)g.e0;  // all -inf: first element
    ChunkOut o;
    o.xmax = xm;
    o.argmax = (MODE == M_ARGMAX) ? ai : -1;
    o.thr = kLowest;
    o.ncand = 0;
    o.s = DO_S ? ss : 0.0;
    o.Rs = DO_S ? RR : kNegInf;
    o.flags = fl;
    if (lane == 0) a.out[(int64_t)g.r * a.nchunks + g.ci] = o;
  }
}

// Truncated rows: a streaming pass that keeps the max of each of the
// thread's NU units (the chunk has at most NU * kTruncBS units, checked by
// the host) and the thread's best unit itself, in registers.  Once t0 is
// known, the units whose max reaches it are candidates; nearly all of them
// are their thread's best, and only the others are read again by their
// lane.  (The streaming loads do not keep the row in L2, so every second
// read is an HBM access: without the kept unit they made 8% more traffic
// than the row on 256 x 6 rows of 128256 bf16 with top-k 50, with it under
// 1%, and the pass went from 67 to 64 us.)
// ALIGNED: the host has checked that V is a multiple of the elements per
// unit, so every chunk starts and ends on a unit boundary and every unit in
// range is whole: the unit code then has one copy per unit (about 40% of
// the code, and fewer registers, against the copy with the edge tests).
template <bool BF16, bool NEED_S, int NU, bool ALIGNED>
__global__ void __launch_bounds__(kTruncBS, 6) trunc_pass_kernel(RowPassArgs a) {
  constexpr int BS = kTruncBS;
  constexpr int EPV = BF16 ? 8 : 4;
  constexpr int NWV = BS / kWave;
  constexpr int kUnroll = NU < 8 ? NU : 8;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const ChunkGeom g = chunk_geom<EPV>(a);
  const uint4* __restrict__ base = reinterpret_cast<const uint4*>(a.logits);
  const float c = a.c;
  if (!g.live) return;

  __shared__ float s_xm[NWV];
  __shared__ double s_s[NWV];
  __shared__ float s_R[NWV];
  __shared__ uint32_t s_fl[NWV], s_kw[NWV];
  __shared__ int s_out;

  // ---- streaming pass: statistics and per-unit maxima ----
  // Unit k of this thread is unit k*BS + tid of the chunk; its first
  // element has the chunk-relative index rel0 + k*BS*EPV (the chunk holds
  // elements [0, n); rel0 >= -(EPV-1)).
  const int n = (int)(g.F1 - g.F0);
  const int nunits = (int)(g.U1 - g.U0);
  const int relu = (int)(g.U0 * EPV - g.F0);  // relative index of unit 0's first element
  const int rel0 = relu + tid * EPV;
  const bool aligned = ALIGNED || ((g.F0 % EPV == 0) && (g.F1 % EPV == 0));
  const int nfull = aligned ? nunits / BS : 0;  // steps whose units are all whole and in range
  UnitAcc<BF16, NEED_S, false> acc;  // the running max is bestv
  float um[NU];
  uint4 bw = make_uint4(0u, 0u, 0u, 0u);
  float bestv = kNegInf;
  int bestk = -1;
#pragma unroll
  for (int k0 = 0; k0 < NU; k0 += kUnroll) {
    uint4 wv[kUnroll];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) wv[i] = ld_stream(base + g.U0 + min((k0 + i) * BS + tid, nunits - 1));
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      const int k = k0 + i;
      const int ul = k * BS + tid;
      const int rel = rel0 + k * BS * EPV;
      float x[EPV];
      um[k] = kNegInf;
      if constexpr (ALIGNED) {
        if (k < nfull || ul < nunits) um[k] = acc.template add<false>(wv[i], rel, n, c, x);
      } else if (k < nfull) {
        um[k] = acc.template add<false>(wv[i], rel, n, c, x);
      } else if (ul < nunits) {
        if (aligned || (ul > 0 && ul + 1 < nunits)) um[k] = acc.template add<false>(wv[i], rel, n, c, x);
        else um[k] = acc.template add<true>(wv[i], rel, n, c, x);
      }
      if (um[k] > bestv) {
        bestv = um[k];
        bestk = k;
        bw = wv[i];
      }
    }
    acc.flush();
  }
  acc.xmax = bestv;
  acc.finish_flags();

  // ---- this wave's ceil(nw/NWV)-th largest thread maximum (bitwise
  //      search on order-preserving keys).  A bf16 value's key ends in 16
  //      equal bits, so the search stops after the upper half: the low half
  //      stays 0, which puts t0 just below that value and no bf16 value in
  //      between, so the same elements reach it. ----
  const int kw = (a.nw + NWV - 1) / NWV;
  const uint32_t tkey = f2key(acc.xmax);
  uint32_t K = 0;
  constexpr int kLowBit = BF16 ? 16 : 0;
  for (int bit = 31; bit >= kLowBit; --bit) {
    const uint32_t cand = K | (1u << bit);
    if ((int)__popcll(ballot(tkey >= cand)) >= kw) K = cand;
  }

  const float wxm = wave_max(acc.xmax);
  const uint32_t wfl = wave_or(acc.flags);
  double ws = acc.s;
  float wR = acc.ref();
  if constexpr (NEED_S) wave_sr_merge(ws, wR);
  if (lane == 0) {
    s_xm[wid] = wxm;
    s_s[wid] = ws;
    s_R[wid] = wR;
    s_fl[wid] = wfl;
    s_kw[wid] = K;
  }
  if (tid == 0) s_out = 0;
  __syncthreads();
  uint32_t t0key = s_kw[0];
  for (int k = 1; k < NWV; ++k) t0key = min(t0key, s_kw[k]);
  t0key = max(t0key, f2key(kLowest));  // -inf logits never become candidates
  const float t0 = key2f(t0key);

  // ---- candidates: every element >= t0 of the units whose max reaches it.
  //      The lane reads such units again, apart from the best unit kept in
  //      registers (units past the chunk have um = -inf < t0).  Places are taken with one LDS atomic per
  //      wave, so the list has no fixed order (the row finisher does not
  //      need one); a list longer than cap_out sends the row to the exact
  //      path. ----
  uint32_t more = 0;  // bit k: unit k (other than the kept best) reaches t0
#pragma unroll
  for (int k = 0; k < NU; ++k) more |= (um[k] >= t0 && k != bestk) ? (1u << k) : 0u;
  Cand* dst = a.cand + ((int64_t)g.r * a.nchunks + g.ci) * a.cap_out;
  const int id0 = (int)g.e0;  // token id of chunk element 0
  uint4 lw[3];
  int lrel[3];
  bool lon[3];
  lw[0] = bw;
  lrel[0] = rel0 + bestk * BS * EPV;
  lon[0] = bestk >= 0 && bestv >= t0;
#pragma unroll
  for (int r = 1; r < 3; ++r) {
    lon[r] = more != 0;
    lrel[r] = 0;
    lw[r] = make_uint4(0u, 0u, 0u, 0u);
    if (lon[r]) {
      const int k = __builtin_ctz(more);
      more &= more - 1;
      lw[r] = base[g.U0 + k * BS + tid];
      lrel[r] = rel0 + k * BS * EPV;
    }
  }
  // Bit e of a unit's mask: element e reaches t0 and lies inside the chunk
  // (elements [max(0, -rel), min(EPV, n - rel)) of the unit do).  The count
  // is the mask's population; the elements are then taken out of the raw
  // 16 bytes by their index, only for the set bits.
  auto unit_mask = [&](const uint4& w, int rel) -> uint32_t {
    float x[EPV];
    widen<BF16>(w, x);
    uint32_t m = 0u;
#pragma unroll
    for (int e = 0; e < EPV; ++e) m |= (x[e] >= t0) ? (1u << e) : 0u;
    const int lo = max(0, -rel), hi = min(EPV, n - rel);
    return hi > lo ? m & ((1u << hi) - (1u << lo)) : 0u;
  };
  // (selects on 64-bit halves, so that the unit stays in registers)
  auto element = [&](uint4 w, int e) -> float {
    const int q = BF16 ? e >> 1 : e;  // 32-bit word of the element
    const uint64_t h = (q & 2) ? (((uint64_t)w.w << 32) | w.z) : (((uint64_t)w.y << 32) | w.x);
    const uint32_t v = (q & 1) ? (uint32_t)(h >> 32) : (uint32_t)h;
    if constexpr (BF16) return __uint_as_float((e & 1) ? (v & 0xffff0000u) : (v << 16));
    else return __uint_as_float(v);
  };
  auto emit_unit = [&](const uint4& w, int rel, uint32_t m, int& pos) {
    while (m != 0u) {
      const int e = __builtin_ctz(m);
      m &= m - 1u;
      if (pos < a.cap_out) {
        Cand ce;
        ce.v = element(w, e);
        ce.idx = id0 + rel + e;
        dst[pos] = ce;
      }
      ++pos;
    }
  };
  uint32_t lm[3];
  int nc = 0;
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    lm[r] = lon[r] ? unit_mask(lw[r], lrel[r]) : 0u;
    nc += __builtin_popcount(lm[r]);
  }
  const int incl = wave_incl_scan_i(nc);
  const int wtot = wave_last_i(incl);
  int wbase = 0;
  if (lane == kWave - 1 && wtot > 0) wbase = atomicAdd(&s_out, wtot);
  wbase = __shfl(wbase, kWave - 1, kWave);
  int pos = wbase + incl - nc;
#pragma unroll
  for (int r = 0; r < 3; ++r) emit_unit(lw[r], lrel[r], lm[r], pos);
  // lanes with more than two further units (ties, flat rows): one at a time
  while (more != 0) {
    const int k = __builtin_ctz(more);
    more &= more - 1;
    const uint4 w = base[g.U0 + k * BS + tid];
    const int rel = rel0 + k * BS * EPV;
    const uint32_t m = unit_mask(w, rel);
    if (m != 0u) {
      int p2 = atomicAdd(&s_out, __builtin_popcount(m));
      emit_unit(w, rel, m, p2);
    }
  }
  __syncthreads();

  // ---- chunk result: wave 0 merges the per-wave partials ----
  if (wid == 0) {
    const bool own = lane < NWV;
    float xm = own ? s_xm[lane] : kNegInf;
    uint32_t fl = own ? s_fl[lane] : 0u;
    double ss = own ? s_s[lane] : 0.0;
    float RR = own ? s_R[lane] : kNegInf;
    xm = wave_max(xm);
    fl = wave_or(fl);
    if constexpr (NEED_S) wave_sr_merge(ss, RR);
    if (lane == 0) {
      int total = s_out;
      if (total > a.cap_out) {
        fl |= CF_OVERFLOW;
        total = a.cap_out;
      }
      ChunkOut o;
      o.xmax = xm;
      o.argmax = -1;
      o.thr = t0;
      o.ncand = total;
      o.s = NEED_S ? ss : 0.0;
      o.Rs = NEED_S ? RR : kNegInf;
      o.flags = fl;
      a.out[(int64_t)g.r * a.nchunks + g.ci] = o;
    }
  }
}

}  // namespace sv
