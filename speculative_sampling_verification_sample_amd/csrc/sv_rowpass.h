// K1 -- the streaming pass over the logits (the HBM-bound hot loop).
//
// Grid nchunks * rows (chunk fastest); each workgroup reads one chunk of one logits row with
// 16-byte loads (8 bf16 or 4 fp32 per load, 64 consecutive loads per wave)
// and produces a ChunkOut:
//   M_SOFTMAX : max and s = sum exp2(x*c - R)   (temperature softmax, [WR] §7.2)
//   M_ARGMAX  : max and the first index holding it    (greedy, [WR] §7.1)
//   M_TRUNC   : max, optional s (top-p needs the full-row mass), and a list of
//               candidates that certainly contains every chunk element >= thr
//               (top-k / top-p, [WR] §7.3).  Candidates are kept in per-wave
//               LDS buffers; a wave whose buffer fills up runs an LDS radix
//               select and keeps its `nw` largest; waves share the highest
//               threshold seen (any wave's nw-th largest is a valid filter for
//               the whole chunk).  At the end the workgroup keeps its `nout`
//               largest (ties included) and writes them out.
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
  int32_t nw;
  int32_t nout;
  int32_t cap_out;
  ChunkOut* out;  // [rows][nchunks]
  Cand* cand;     // [rows][nchunks][cap_out]
  // Optional draft gather (untruncated sampling): the workgroup whose chunk
  // holds d_j stores (z(d_j), q_j(d_j)) in gath[row].
  const int32_t* ids;
  const float* q;
  int32_t gamma;
  float2* gath;
};

constexpr int kCapW = 512;  // candidate slots per wave

// Radix select inside one wave: the key of the `need`-th largest entry.
template <bool BF16>
__device__ uint32_t wave_select(const Cand* buf, int cnt, int need, uint32_t* hist) {
  const int lane = lane_id();
  uint32_t prefix = 0, pmask = 0;
  constexpr int kLow = BF16 ? 16 : 0;
  for (int shift = 24; shift >= kLow; shift -= 8) {
    for (int k = lane; k < 256; k += kWave) hist[k] = 0;
    wave_sync();
    for (int i = lane; i < cnt; i += kWave) {
      uint32_t key = f2key(buf[i].v);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    wave_sync();
    int digit = wave_find_digit(hist, need);
    prefix |= (uint32_t)digit << shift;
    pmask |= 255u << shift;
    wave_sync();
  }
  return prefix;
}

// Keep entries with key >= K (in place, order preserved); returns the count.
__device__ int wave_filter(Cand* buf, int cnt, uint32_t K) {
  const int lane = lane_id();
  int newcnt = 0;
  for (int base = 0; base < cnt; base += kWave) {
    int i = base + lane;
    bool valid = i < cnt;
    Cand e;
    e.v = kNegInf;
    e.idx = 0;
    if (valid) e = buf[i];
    bool keep = valid && f2key(e.v) >= K;
    uint64_t m = ballot(keep);
    wave_sync();
    if (keep) buf[newcnt + lanes_below(m)] = e;
    newcnt += (int)__popcll(m);
    wave_sync();
  }
  return newcnt;
}

template <int MODE, bool BF16, bool NEED_S, int BS>
__global__ void __launch_bounds__(BS) rowpass_kernel(RowPassArgs a) {
  constexpr int EPV = BF16 ? 8 : 4;
  constexpr int NWV = BS / kWave;
  constexpr bool DO_S = (MODE == M_SOFTMAX) || NEED_S;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int64_t blk = blockIdx.x;  // linear grid, chunk index fastest
  const int r = (int)(blk / a.nchunks), ci = (int)(blk - (int64_t)r * a.nchunks);
  const int b = r / a.rows_per_req, j = r - b * a.rows_per_req;
  const int64_t rowoff = ((int64_t)b * a.G1 + j) * a.V;
  const int64_t e0 = (int64_t)ci * a.chunk;
  const int64_t e1 = min(e0 + a.chunk, a.V);
  const int64_t F0 = rowoff + e0, F1 = rowoff + e1;
  const int64_t U0 = F0 / EPV, U1 = (F1 + EPV - 1) / EPV;
  const uint4* __restrict__ base = reinterpret_cast<const uint4*>(a.logits);
  const float c = a.c;

  __shared__ uint32_t s_thr;  // shared candidate threshold (key), monotone
  __shared__ int s_cnt[NWV];
  __shared__ float s_xm[NWV];
  __shared__ int s_ai[NWV];
  __shared__ double s_s[NWV];
  __shared__ float s_R[NWV];
  __shared__ uint32_t s_fl[NWV];
  __shared__ uint32_t s_hist[256];
  __shared__ int s_digit, s_need, s_out;
  extern __shared__ __align__(16) unsigned char s_dyn[];

  Cand* wbuf = nullptr;
  uint32_t* whist = nullptr;
  if constexpr (MODE == M_TRUNC) {
    wbuf = reinterpret_cast<Cand*>(s_dyn) + wid * kCapW;
    whist = reinterpret_cast<uint32_t*>(s_dyn + (size_t)NWV * kCapW * sizeof(Cand)) + wid * 256;
    if (tid == 0) s_thr = f2key(kLowest);
    __syncthreads();
  }

  if (a.gath != nullptr && tid == 0 && j < a.gamma) {
    const int d = a.ids[(int64_t)b * a.gamma + j];
    if ((int64_t)d >= e0 && (int64_t)d < e1) {
      float zd = BF16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(a.logits)[rowoff + d] << 16)
                      : reinterpret_cast<const float*>(a.logits)[rowoff + d];
      a.gath[r] = make_float2(zd, a.q[((int64_t)b * a.gamma + j) * a.V + d]);
    }
  }

  float xmax = kNegInf;
  int64_t bestu = -1;
  double s = 0.0;
  float R = kNegInf;
  uint32_t nan_words = 0;  // max of |bits| over full units (per 16-bit half for bf16)
  uint32_t flags = 0;
  // TRUNC state (wave-uniform)
  int cnt = 0;
  float thr = kLowest;
  bool dead = false;

  auto compact = [&]() {
    uint32_t K = wave_select<BF16>(wbuf, cnt, a.nw, whist);
    cnt = wave_filter(wbuf, cnt, K);
    if (lane == 0) atomicMax(&s_thr, K);
    wave_sync();
    uint32_t Ks = max(K, __atomic_load_n(&s_thr, __ATOMIC_RELAXED));
    thr = key2f(Ks);
    if (cnt > kCapW - kWave) dead = true;  // ties alone fill the buffer
  };

  auto process = [&](int64_t u, const uint4& w, auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    float x[EPV];
    widen<BF16>(w, x);
    if constexpr (EDGE) {
#pragma unroll
      for (int i = 0; i < EPV; ++i) {
        int64_t f = u * EPV + i;
        if (f < F0 || f >= F1) x[i] = kNegInf;
        else if (x[i] != x[i]) flags |= CF_NAN;
      }
    } else if constexpr (!DO_S) {
      // no exp sums in this mode: NaN needs its own test (|bits| above +Inf)
      if constexpr (BF16) {
        uint32_t m0 = w.x & 0x7fff7fffu, m1 = w.y & 0x7fff7fffu, m2 = w.z & 0x7fff7fffu, m3 = w.w & 0x7fff7fffu;
        uint32_t lo = max(max(m0 & 0xffffu, m1 & 0xffffu), max(m2 & 0xffffu, m3 & 0xffffu));
        uint32_t hi = max(max(m0 >> 16, m1 >> 16), max(m2 >> 16, m3 >> 16));
        nan_words = max(nan_words, max(lo, hi));
      } else {
        uint32_t m = max(max(w.x & 0x7fffffffu, w.y & 0x7fffffffu), max(w.z & 0x7fffffffu, w.w & 0x7fffffffu));
        nan_words = max(nan_words, m);
      }
    }
    float vm = x[0];
#pragma unroll
    for (int i = 1; i < EPV; ++i) vm = fmaxf(vm, x[i]);
    if constexpr (MODE == M_ARGMAX) {
      if (vm > xmax) {
        xmax = vm;
        bestu = u;
      }
    } else {
      xmax = fmaxf(xmax, vm);
    }
    if constexpr (DO_S) {
      float vc = vm * c;
      if (vc > R && vm < kPosInf) {
        float Rn = ceilf(vc);
        if (R != kNegInf) s = ldexp(s, (int)(R - Rn));
        R = Rn;
      }
      if (R != kNegInf) {
        // a NaN logit turns s into NaN, which the row merge reports
        float ev[EPV];
#pragma unroll
        for (int i = 0; i < EPV; ++i) ev[i] = e_of(x[i], c, R);
        float t;
        if constexpr (EPV == 8) t = ((ev[0] + ev[1]) + (ev[2] + ev[3])) + ((ev[4] + ev[5]) + (ev[6] + ev[7]));
        else t = (ev[0] + ev[1]) + (ev[2] + ev[3]);
        s += (double)t;
      } else {
        // nothing finite seen yet by this thread: test this unit directly
#pragma unroll
        for (int i = 0; i < EPV; ++i)
          if (x[i] != x[i]) flags |= CF_NAN;
      }
    }
    if constexpr (MODE == M_TRUNC) {
      if (ballot(vm >= thr) != 0 && !dead) {
#pragma unroll
        for (int i = 0; i < EPV; ++i) {
          if (cnt > kCapW - kWave) {
            compact();
            if (dead) break;
          }
          bool p = x[i] >= thr;
          uint64_t m = ballot(p);
          if (p) {
            Cand e;
            e.v = x[i];
            e.idx = (int32_t)(u * EPV + i - rowoff);
            wbuf[cnt + lanes_below(m)] = e;
          }
          cnt += (int)__popcll(m);
        }
      }
    }
  };

  using Edge = std::true_type;
  using NoEdge = std::false_type;

  // Block-uniform steps: step k gives thread tid the unit U0 + k*BS + tid.
  // Every thread runs every step (lanes past the end see an all -inf unit),
  // so the wave-wide ballots and LDS selections of M_TRUNC see whole waves.
  // Up to kUnroll units' loads are issued before any is processed.
  constexpr int kUnroll = 8;
  const bool aligned = (F0 % EPV == 0) && (F1 % EPV == 0);
  const int64_t nunits = U1 - U0;
  const int64_t nsteps = (nunits + BS - 1) / BS;
  const int64_t nfull = aligned ? nunits / BS : 0;  // steps whose units are all whole and in range
  for (int64_t k0 = 0; k0 < nsteps; k0 += kUnroll) {
    uint4 wv[kUnroll];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      const int64_t u = U0 + (k0 + i) * BS + tid;
      wv[i] = make_uint4(0u, 0u, 0u, 0u);
      if (k0 + i < nsteps && u < U1) wv[i] = base[u];
    }
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      if (k0 + i >= nsteps) break;
      const int64_t u = U0 + (k0 + i) * BS + tid;
      if (k0 + i < nfull) process(u, wv[i], NoEdge{});
      else process(u, wv[i], Edge{});
    }
  }

  // NaN / +Inf detection
  if constexpr (BF16) {
    if (nan_words > 0x7f80u) flags |= CF_NAN;
  } else {
    if (nan_words > 0x7f800000u) flags |= CF_NAN;
  }
  if (xmax == kPosInf) flags |= CF_POSINF;

  // ---- argmax index inside the best unit ----
  int aidx = 0x7fffffff;
  if constexpr (MODE == M_ARGMAX) {
    if (bestu >= 0) {
      uint4 w = base[bestu];
      float x[EPV];
      widen<BF16>(w, x);
#pragma unroll
      for (int i = EPV - 1; i >= 0; --i) {
        int64_t f = bestu * EPV + i;
        if (f >= F0 && f < F1 && x[i] == xmax) aidx = (int)(f - rowoff);
      }
    }
  }

  // ---- workgroup reductions (fixed order) ----
  float wxm = xmax;
  int wai = aidx;
  if constexpr (MODE == M_ARGMAX) wave_argmax(wxm, wai);
  else wxm = wave_max(wxm);
  if (MODE == M_TRUNC && dead) flags |= CF_OVERFLOW;
  uint32_t wfl = wave_or(flags);
  double ws = s;
  float wR = R;
  if constexpr (DO_S) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      double s2 = __shfl_xor(ws, o, kWave);
      float R2 = __shfl_xor(wR, o, kWave);
      sr_merge(ws, wR, s2, R2);
    }
  }
  if (lane == 0) {
    s_xm[wid] = wxm;
    s_ai[wid] = wai;
    s_s[wid] = ws;
    s_R[wid] = wR;
    s_fl[wid] = wfl;
  }

  if constexpr (MODE == M_TRUNC) {
    // Final candidate set of the chunk.
    __syncthreads();
    uint32_t Ks = s_thr;
    cnt = wave_filter(wbuf, cnt, Ks);
    if (lane == 0) s_cnt[wid] = cnt;
    __syncthreads();
    int total = 0;
    for (int k = 0; k < NWV; ++k) total += s_cnt[k];
    uint32_t Kc = Ks;
    if (total > a.nout) {
      uint32_t prefix = 0, pmask = 0;
      int need = a.nout;
      constexpr int kLow = BF16 ? 16 : 0;
      for (int shift = 24; shift >= kLow; shift -= 8) {
        if (tid < 256) s_hist[tid] = 0;
        __syncthreads();
        for (int i = lane; i < cnt; i += kWave) {
          uint32_t key = f2key(wbuf[i].v);
          if ((key & pmask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (wid == 0) {
          int d = wave_find_digit(s_hist, need);
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
      Kc = prefix;
    }
    if (tid == 0) s_out = 0;
    __syncthreads();
    Cand* dst = a.cand + ((int64_t)r * a.nchunks + ci) * a.cap_out;
    for (int bse = 0; bse < cnt; bse += kWave) {
      int i = bse + lane;
      bool keep = i < cnt && f2key(wbuf[i].v) >= Kc;
      uint64_t m = ballot(keep);
      int basepos = 0;
      if (lane == 0 && m) basepos = atomicAdd(&s_out, (int)__popcll(m));
      basepos = __shfl(basepos, 0, kWave);
      int pos = basepos + lanes_below(m);
      if (keep && pos < a.cap_out) dst[pos] = wbuf[i];
    }
    __syncthreads();
    if (tid == 0) {
      ChunkOut o;
      float xm = s_xm[0];
      uint32_t fl = s_fl[0];
      double ss = s_s[0];
      float RR = s_R[0];
      for (int k = 1; k < NWV; ++k) {
        xm = fmaxf(xm, s_xm[k]);
        fl |= s_fl[k];
        if constexpr (NEED_S) sr_merge(ss, RR, s_s[k], s_R[k]);
      }
      int no = s_out;
      if (no > a.cap_out) {
        fl |= CF_OVERFLOW;
        no = a.cap_out;
      }
      o.xmax = xm;
      o.argmax = -1;
      o.thr = key2f(Kc);
      o.ncand = no;
      o.s = NEED_S ? ss : 0.0;
      o.Rs = NEED_S ? RR : kNegInf;
      o.flags = fl;
      a.out[(int64_t)r * a.nchunks + ci] = o;
    }
  } else {
    __syncthreads();
    if (tid == 0) {
      float xm = s_xm[0];
      int ai = s_ai[0];
      uint32_t fl = s_fl[0];
      double ss = s_s[0];
      float RR = s_R[0];
      for (int k = 1; k < NWV; ++k) {
        if constexpr (MODE == M_ARGMAX) argmax_merge(xm, ai, s_xm[k], s_ai[k]);
        else xm = fmaxf(xm, s_xm[k]);
        fl |= s_fl[k];
        if constexpr (DO_S) sr_merge(ss, RR, s_s[k], s_R[k]);
      }
      if (MODE == M_ARGMAX && xm == kNegInf) ai = (int)e0;  // all -inf: first element
      ChunkOut o;
      o.xmax = xm;
      o.argmax = (MODE == M_ARGMAX) ? ai : -1;
      o.thr = kLowest;
      o.ncand = 0;
      o.s = DO_S ? ss : 0.0;
      o.Rs = DO_S ? RR : kNegInf;
      o.flags = fl;
      a.out[(int64_t)r * a.nchunks + ci] = o;
    }
  }
}

}  // namespace sv
