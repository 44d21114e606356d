// C-ABI front end: argument validation, the shape-only plan, workspace
// layout and the launch on the caller's stream.  See include/mgqa.h for the
// contract of every entry point.
#include "mgqa.h"

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "mgqa_internal.h"

namespace mgqa {
namespace {

constexpr int kCUs = 256;              // MI355X compute units
// Split-KV path: position blocks and key splits are chosen so that about this
// many workgroups run.
constexpr long long kSplitTarget = 256;
constexpr int kMaxCounters = 256;  // leading counter block
static_assert(kSplitTarget <= kMaxCounters, "split plans need one counter per group");
// Splits of one key band from which two column halves pay off.
constexpr long long kHalfColumnsMinSplits = 8;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Largest K/V unit (one batch row and kv head: Lkv*d or S*d elements).  The
// kernels address a unit through a buffer descriptor with 32-bit byte offsets
// and use byte offset 2^31 as "outside every range" (a zero read), so a unit
// may span at most 2^31 bytes.
constexpr long long kMaxUnitElems = 1LL << 30;

int validate(int B, int Hq, int Hkv, int Lq, int Lkv, int d, int causal, int window,
             float softcap, int dtype) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lq <= 0 || Lkv <= 0 || d <= 0) return MGQA_ERR_SHAPE;
  if (Hq % Hkv != 0 || Hq / Hkv > 16) return MGQA_ERR_SHAPE;
  if (d % 8 != 0 || d > 128) return MGQA_ERR_HEAD_DIM;
  if (causal != 0 && causal != 1) return MGQA_ERR_MASK;
  if (window < 0) return MGQA_ERR_MASK;
  if ((causal || window > 0) && Lq > Lkv) return MGQA_ERR_MASK;
  if (!(softcap >= 0.f) || isinf(softcap)) return MGQA_ERR_SOFTCAP;  // also rejects NaN
  if (dtype != MGQA_BF16 && dtype != MGQA_FP16) return MGQA_ERR_DTYPE;
  // 32-bit indexing inside the kernels: per-tensor element counts and grid size.
  const long long q_elems = (long long)B * Hq * Lq * d;
  const long long kv_elems = (long long)B * Hkv * Lkv * d;
  if (q_elems > (1LL << 40) || kv_elems > (1LL << 40)) return MGQA_ERR_RANGE;
  if ((long long)Lkv * d > kMaxUnitElems || (long long)Lq * Hq >= (1LL << 31)) return MGQA_ERR_RANGE;
  return MGQA_OK;
}

}  // namespace

// Key band [lo, hi] of the query positions [q0, q0 + m_eff) (bottom-right aligned).
static void block_band(int q0, int m_eff, int Lq, int Lkv, int causal, int window, int* lo, int* hi) {
  const int off = Lkv - Lq;
  const int pos_min = q0 + off, pos_max = q0 + m_eff - 1 + off;
  *lo = 0;
  *hi = Lkv - 1;
  if (causal && pos_max < *hi) *hi = pos_max;
  if (window > 0) {
    if (pos_min - window + 1 > 0) *lo = pos_min - window + 1;
    if (!causal && pos_max + window - 1 < *hi) *hi = pos_max + window - 1;
  }
}

// ---------------------------------------------------------------------------
// Work items of the pipelined head-size-128 prefill kernel.  A launch runs in
// rounds of 512 workgroups (two per CU); its length is set by the last round.
// Under a causal mask the first position blocks (the ramp) have shorter key
// bands than the rest; taken last first they leave a last round of short
// blocks that finishes long after the average.  Two remedies, chosen by a
// model of the launch: the two ends of the ramp paired into one workgroup
// (blocks R-1-j and j: about one full band together), and the last round
// filled with half blocks (64 rows) instead of part-filled with whole ones.
// ---------------------------------------------------------------------------
namespace {

// Model of a launch, in 32-key steps of a 128-row block taken by one of two
// workgroups sharing a CU.  A block costs kPipeSetupSteps of set-up (Q loads,
// the first tiles' round trip, the output) plus one step per tile of its
// band; a 64-row half block kPipeHalfStep per tile.  A workgroup alone on
// its CU runs kPipeAloneSpeed times faster.  (Fitted to timings of causal and
// windowed prefill launches on MI355X.)
constexpr double kPipeSetupSteps = 4.0;
constexpr double kPipeHalfStep = 0.7;
constexpr double kPipeAloneSpeed = 1.6;
constexpr int kXCDs = 8;
constexpr int kCUsPerXCD = kCUs / kXCDs;
constexpr long long kPipeMaxModeled = 1 << 18;  // larger grids keep the plain order

struct PipeSched {
  int items, pairs, ramp, full;
};

int band_tiles(int q0, int m, int Lq, int Lkv, int causal, int window) {
  int lo, hi;
  block_band(q0, Lq - q0 < m ? Lq - q0 : m, Lq, Lkv, causal, window, &lo, &hi);
  return hi / kPipe4Keys - lo / kPipe4Keys + 1;
}

// Modeled length of the launch.  Every XCD starts its workgroups in order,
// each on the least occupied of its CUs that has room (two per CU).  With a
// grid that is a multiple of 8 the kernel gives XCD x the x-th eighth of the
// (unit, item) list; otherwise the hardware deals workgroup i to XCD i % 8.
double pipe_makespan(const PipeSched& s, long long units, const std::vector<int>& tiles, int m, int Lq,
                     int Lkv, int causal, int window) {
  const int n = (int)tiles.size();
  std::vector<double> cost(s.items);
  for (int j = 0; j < s.items; ++j) {
    if (j < s.pairs) {
      const int hi = s.ramp - 1 - j;
      cost[j] = kPipeSetupSteps + tiles[hi] + (j < hi ? kPipeSetupSteps + tiles[j] : 0.0);
    } else if (j < s.pairs + s.full) {
      cost[j] = kPipeSetupSteps + tiles[n - 1 - (j - s.pairs)];
    } else {
      const int h = j - s.pairs - s.full, pb = n - 1 - s.full - (h >> 1);
      const int q0 = pb * m + (h & 1) * (m / 2);
      cost[j] = kPipeSetupSteps + kPipeHalfStep * band_tiles(q0, m / 2, Lq, Lkv, causal, window);
    }
  }
  const long long nwg = units * s.items;
  const bool renumbered = nwg % kXCDs == 0;
  double worst = 0.0;
  double rem[kCUsPerXCD][2];  // work left in each slot (0: free)
  int busy[kCUsPerXCD];
  for (int x = 0; x < kXCDs; ++x) {
    const long long first = renumbered ? x * (nwg / kXCDs) : x;
    const long long stop = renumbered ? (x + 1) * (nwg / kXCDs) : nwg;
    const long long stride = renumbered ? 1 : kXCDs;
    for (int c = 0; c < kCUsPerXCD; ++c) rem[c][0] = rem[c][1] = 0.0, busy[c] = 0;
    long long next = first;
    double t = 0.0;
    int running = 0;
    while (true) {
      // Start workgroups while a CU has room: empty CUs first.
      while (next < stop) {
        int best = -1;
        for (int c = 0; c < kCUsPerXCD && best < 0; ++c)
          if (busy[c] == 0) best = c;
        for (int c = 0; c < kCUsPerXCD && best < 0; ++c)
          if (busy[c] == 1) best = c;
        if (best < 0) break;
        const int slot = rem[best][0] > 0.0 ? 1 : 0;
        rem[best][slot] = cost[next % s.items];
        ++busy[best];
        ++running;
        next += stride;
      }
      if (running == 0) break;
      // Advance to the next completion.
      double dt = 1e300;
      for (int c = 0; c < kCUsPerXCD; ++c) {
        const double speed = busy[c] == 1 ? kPipeAloneSpeed : 1.0;
        for (int k = 0; k < 2; ++k)
          if (rem[c][k] > 0.0) dt = std::min(dt, rem[c][k] / speed);
      }
      t += dt;
      for (int c = 0; c < kCUsPerXCD; ++c) {
        const double speed = busy[c] == 1 ? kPipeAloneSpeed : 1.0;
        for (int k = 0; k < 2; ++k)
          if (rem[c][k] > 0.0) {
            rem[c][k] -= dt * speed;
            if (rem[c][k] <= 1e-9) {
              rem[c][k] = 0.0;
              --busy[c];
              --running;
            }
          }
      }
    }
    worst = std::max(worst, t);
    if (renumbered && units % kXCDs == 0) break;  // every XCD runs the same list
  }
  return worst;
}

PipeSched pipe_schedule_uncached(long long units, int n, int m, int Lq, int Lkv, int causal, int window) {
  const PipeSched plain = {n, 0, 0, n};
  if (units * n > kPipeMaxModeled) return plain;
  std::vector<int> tiles(n);
  int tmax = 0;
  for (int pb = 0; pb < n; ++pb) {
    tiles[pb] = band_tiles(pb * m, m, Lq, Lkv, causal, window);
    tmax = std::max(tmax, tiles[pb]);
  }
  // Ramp: the leading blocks whose band is shorter than the longest by two
  // tiles or more (bands of the full blocks differ by one tile with their
  // alignment).
  int ramp = 0;
  if (causal)
    while (ramp < n && tiles[ramp] < tmax - 1) ++ramp;
  // The last block, when partial, is never halved: its second half could be
  // empty.
  const int keep = (Lq % m != 0) ? 1 : 0;
  PipeSched best = plain;
  double best_t = pipe_makespan(plain, units, tiles, m, Lq, Lkv, causal, window);
  const double plain_t = best_t;
  // Without pairs (r = 0), and with the ramp's ends paired (r = ramp).
  // Candidates: the ramp's ends paired (r = ramp) or not (r = 0), each with
  // no half blocks, with as many as turn the part-filled last round of whole
  // blocks into a round of halves, and (without pairs) every block halved.
  const int nr = ramp >= 2 ? 2 : 1;
  for (int c = 0; c < nr; ++c) {
    const int r = c ? ramp : 0;
    const int pairs = (r + 1) / 2;
    const int blocks = n - r;  // whole blocks past the ramp
    const int hmax = (m % 2 == 0) ? blocks - keep : 0;
    auto eval = [&](int H) {
      if (H < 0 || H > hmax || (r == 0 && H == 0)) return;  // (r, H) = (0, 0) is the plain order
      const PipeSched s = {pairs + blocks + H, pairs, r, blocks - H};
      const double t = pipe_makespan(s, units, tiles, m, Lq, Lkv, causal, window);
      if (t < best_t) {
        best_t = t;
        best = s;
      }
    };
    eval(0);
    const long long round = 2LL * kCUs;
    const long long rest = (units * (pairs + blocks)) % round;
    if (rest > 0) eval((int)((rest + units - 1) / units));
    if (r == 0 && units * blocks <= round) eval(hmax);
  }
  // Keep the plain order unless the model gains at least 2%.
  return best_t < 0.98 * plain_t ? best : plain;
}

PipeSched pipe_schedule(long long units, int n, int m, int Lq, int Lkv, int causal, int window) {
  // A few recent shapes per thread: repeated calls of one shape plan once.
  constexpr int kMemo = 8;
  struct Entry {
    long long key[7];
    PipeSched s;
  };
  thread_local Entry memo[kMemo];
  thread_local int filled = 0, next = 0;
  const long long k[7] = {units, n, m, Lq, Lkv, causal, window};
  for (int i = 0; i < filled; ++i)
    if (std::equal(k, k + 7, memo[i].key)) return memo[i].s;
  Entry& e = memo[next];
  std::copy(k, k + 7, e.key);
  e.s = pipe_schedule_uncached(units, n, m, Lq, Lkv, causal, window);
  next = (next + 1) % kMemo;
  if (filled < kMemo) ++filled;
  return e.s;
}

}  // namespace

// Largest number of 32-key steps in the key band of any block of m query
// positions, or any number above `limit` once one block exceeds it.
static int max_block_steps(int m, int Lq, int Lkv, int causal, int window, int limit) {
  // A block's band spans at most m - 1 + window keys under a causal window,
  // m - 1 + 2*window - 1 under a two-sided one, and Lkv keys in any case;
  // 32-key steps over a span of n keys: at most (n + 30) / 32 + 1.
  long long span = Lkv;
  if (window > 0) span = std::min<long long>(span, (long long)m - 1 + (causal ? window : 2LL * window - 1));
  if ((span + 30) / 32 + 1 <= limit) return (int)((span + 30) / 32 + 1);
  int worst = 1;
  for (int q0 = 0; q0 < Lq; q0 += m) {
    int lo, hi;
    block_band(q0, Lq - q0 < m ? Lq - q0 : m, Lq, Lkv, causal, window, &lo, &hi);
    const int steps = hi / 32 - lo / 32 + 1;
    if (steps > worst) worst = steps;
    if (worst > limit) break;
  }
  return worst;
}

int make_plan(int B, int Hq, int Hkv, int Lq, int Lkv, int d, int causal, int window,
              float softcap, int dtype, Plan* plan) {
  const int err = validate(B, Hq, Hkv, Lq, Lkv, d, causal, window, softcap, dtype);
  if (err) return err;
  Plan p = {};
  const int G = Hq / Hkv;
  p.dqk = (d + 31) / 32;
  p.qk_pad = 32 * p.dqk;
  p.dv = (d <= 80 && d > 64) ? 5 : 2 * p.dqk;  // 72 and 80 use a 80-wide P.V
  const long long units = (long long)B * Hkv;
  const long long rows_all = (long long)G * Lq;
  const int max_nqb = p.dv <= kSplitWideMaxDv ? kSplitMaxNqb : kSplitMaxNqbWide;

  // Prefill kernels: 256-row blocks (128-row blocks, two workgroups per CU,
  // for head size 128; 128-row blocks of one 16-row block per wave for head
  // sizes 104-120), when that still gives a workgroup per CU.
  const bool d128 = (d == 128);
  const int pf_nqb = (!d128 && p.dqk == 4) ? kPrefillNqbWide : kPrefillNqb;
  const int rows_big = d128 ? 16 * kPipe4Waves * kPrefillNqb : 16 * kPrefillWaves * pf_nqb;
  const int m_big = rows_big / G;
  const long long wgs_big = units * ((Lq + m_big - 1) / m_big);
  if (rows_all > 16LL * max_nqb && wgs_big >= kCUs) {
    p.path = kPathPrefill;
    p.keys_per_tile = d128 ? kPipe4Keys : kPrefillKeys;
    p.nsplit = 1;
    p.nqb = pf_nqb;
    p.nwaves = d128 ? kPipe4Waves : kPrefillWaves;
    p.rows_per_wg = 16 * p.nwaves * p.nqb;
    p.m = m_big;
    p.n_pos_blk = (Lq + m_big - 1) / m_big;
    PipeSched s = {p.n_pos_blk, 0, 0, p.n_pos_blk};
    if (d128) s = pipe_schedule(units, p.n_pos_blk, p.m, Lq, Lkv, causal, window);
    p.pf_items = s.items;
    p.pf_pairs = s.pairs;
    p.pf_ramp = s.ramp;
    p.pf_full = s.full;
    p.workgroups = units * s.items;
    if (p.workgroups >= (1LL << 31)) return MGQA_ERR_RANGE;
    *plan = p;
    return MGQA_OK;
  }

  // Split-KV kernel.  Every row in one workgroup when they fit (decode and
  // multi-token decode: K/V are read once per unit); otherwise the largest
  // row block that still gives a workgroup per CU.  Then the key band is split
  // across workgroups until about one workgroup per CU runs.
  p.path = kPathSplit;
  p.keys_per_tile = kSplitKeys;
  p.nwaves = kSplitWaves;
  bool short_band = false;
  if (rows_all <= 16LL * max_nqb) {
    p.nqb = (int)((rows_all + 15) / 16);
    p.m = Lq;
  } else if (d > 48 && d <= 96 && max_block_steps(16 * kEncNqb / G, Lq, Lkv, causal, window, kEncMaxSteps) <= kEncMaxSteps) {
    // Short bands (at most kEncMaxSteps 32-key steps for a block of 48/G
    // positions), head size 49..96: the short-band kernel, whatever the
    // workgroup count.  Its eight waves split the band among themselves and
    // merge in LDS; on the 729-token encoder with 1 to 8 heads this was
    // faster than key splits across workgroups (4 heads: 8.5 against 10.6 us).
    short_band = true;
    p.nqb = kEncNqb;
    p.m = 16 * kEncNqb / G;
  } else {
    p.nqb = 1;
    for (int nqb = max_nqb; nqb >= 1; --nqb) {
      const int m = 16 * nqb / G;
      if (m >= 1 && units * ((Lq + m - 1) / m) >= kSplitTarget) {
        p.nqb = nqb;
        break;
      }
    }
    p.m = 16 * p.nqb / G;
  }
  p.rows_per_wg = 16 * p.nqb;
  p.n_pos_blk = (Lq + p.m - 1) / p.m;
  const long long groups = units * p.n_pos_blk;
  // Largest band of any position block, in tiles of `keys` keys.
  auto max_band_tiles = [&](int keys) {
    int max_tiles = 1;
    for (int pb = 0; pb < p.n_pos_blk; ++pb) {
      const int q0 = pb * p.m;
      const int m_eff = Lq - q0 < p.m ? Lq - q0 : p.m;
      int lo, hi;
      block_band(q0, m_eff, Lq, Lkv, causal, window, &lo, &hi);
      const int tiles = hi / keys - lo / keys + 1;
      if (tiles > max_tiles) max_tiles = tiles;
    }
    return max_tiles;
  };
  long long ns = 1;
  int tps = 1 << 30;  // one split: the whole band
  int ncol = 1;
  if (groups < kSplitTarget && !short_band) {
    const int max_tiles = max_band_tiles(kSplitKeys);
    ns = (kSplitTarget + groups - 1) / groups;
    if (ns > max_tiles) ns = max_tiles;
    // Column halves: with many splits of one 16-row block the last arrival
    // reads nsplit partials of the whole head size.  Two workgroups per key
    // range, each with half of V's columns, halve both the number of splits
    // and the width of each partial (a quarter of the merge reads), for the
    // same workgroup count; the pair reads the same K rows at the same time
    // on one XCD, so K comes from HBM once.
    if (ns >= kHalfColumnsMinSplits && p.dv == 8 && p.nqb == 1 && groups * 2 <= kMaxCounters) {
      ncol = 2;
      ns = (kSplitTarget + 2 * groups - 1) / (2 * groups);
      if (ns > max_tiles) ns = max_tiles;
    }
    tps = (int)((max_tiles + ns - 1) / ns);
    ns = (max_tiles + tps - 1) / tps;
  }
  // Wide workgroups: a single 16-row block with a long key range per
  // workgroup streams 256-key tiles with 8 waves (two per SIMD), twice the
  // bytes in flight per workgroup, for the same splits.
  if (p.nqb == 1 && ncol == 1 && (ns > 1 ? tps : max_band_tiles(kSplitKeys)) >= kSplitWideMinTiles) {
    p.nwaves = kSplitWavesWide;
    p.keys_per_tile = 32 * kSplitWavesWide;
    if (ns > 1) {
      const int max_tiles = max_band_tiles(p.keys_per_tile);
      tps = (int)((max_tiles + ns - 1) / ns);
      ns = (max_tiles + tps - 1) / tps;
    }
  }
  // The short-band kernel: eight waves that each take their own contiguous
  // keys of a band of at most 768 keys (head size 49..96).  Chosen above for
  // blocks of 48 rows; also taken by the rows of a multi-token step that fill
  // three 16-row blocks when the band is left unsplit.
  if (!short_band && p.nqb == kEncNqb && ns == 1 && d > 48 && d <= 96 && max_band_tiles(32) <= kEncMaxSteps)
    short_band = true;
  if (short_band) {
    p.path = kPathShort;
    p.nwaves = kEncWaves;
    p.keys_per_tile = 32 * kEncSteps;  // the most keys one wave takes
  }
  p.nsplit = (int)ns;
  p.tiles_per_split = tps;
  p.ncol = ns > 1 ? ncol : 1;
  p.workgroups = groups * ns * p.ncol;
  if (ns > 1) {
    const size_t nrows = (size_t)p.m * G;
    const size_t o_bytes = (size_t)groups * ns * nrows * (p.dv * 16) * sizeof(float);
    const size_t ml_bytes = (size_t)groups * p.ncol * ns * nrows * 2 * sizeof(float);
    // Key splits happen only with fewer than kSplitTarget groups, so the
    // counters of every plan fit the same leading kMaxCounters words: no plan
    // writes partials there, and the counters a call leaves at zero stay zero
    // for the next call on the same workspace, whatever its shape.
    p.ws_cnt_off = 0;
    p.ws_ml_off = align_up((size_t)kMaxCounters * sizeof(unsigned), 256);
    p.ws_o_off = align_up(p.ws_ml_off + ml_bytes, 256);
    p.ws_bytes = align_up(p.ws_o_off + o_bytes, 256);
  }
  if (p.workgroups >= (1LL << 31)) return MGQA_ERR_RANGE;
  if (ns > 1 && groups * p.ncol > kMaxCounters) return MGQA_ERR_RANGE;  // cannot happen: see the counter layout
  // 32-bit byte offsets of the partials inside the kernel.
  if (p.ws_bytes >= (1ULL << 31)) return MGQA_ERR_RANGE;
  *plan = p;
  return MGQA_OK;
}

static KernelArgs make_args(const Plan& p, const void* q, const void* k, const void* v, void* out,
                            int Hq, int Hkv, int Lq, int Lkv, int d, int causal, int window,
                            float softcap, void* ws) {
  KernelArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.Lq = Lq;
  a.Lkv = Lkv;
  a.d = d;
  a.kv_stride = (long long)Lkv * d;
  a.ring_start = -1;
  a.ring_slots = Lkv;
  a.causal = causal;
  a.window = window;
  const double log2e = 1.4426950408889634;
  a.alpha = (float)(log2e / sqrt((double)d));
  if (softcap > 0.f) {
    a.gamma = (float)(2.0 * log2e / ((double)softcap * sqrt((double)d)));
    a.c2 = (float)((double)softcap * log2e);
    a.beta = (float)(1.0 / ((double)softcap * sqrt((double)d)));
  }
  a.m = p.m;
  a.n_pos_blk = p.n_pos_blk;
  a.nsplit = p.nsplit;
  a.div_g = make_fastdiv((uint32_t)a.G);
  a.div_hkv = make_fastdiv((uint32_t)Hkv);
  a.div_npos = make_fastdiv((uint32_t)p.n_pos_blk);
  a.div_nsplit = make_fastdiv((uint32_t)p.nsplit);
  a.nwg = (int)p.workgroups;
  a.tiles_per_split = p.tiles_per_split;
  a.nrows = p.m * a.G;
  a.pf_items = p.pf_items;
  a.pf_pairs = p.pf_pairs;
  a.pf_ramp = p.pf_ramp;
  a.pf_full = p.pf_full;
  a.div_items = make_fastdiv((uint32_t)(p.pf_items > 0 ? p.pf_items : 1));
  if (ws) {
    char* base = static_cast<char*>(ws);
    a.ws_cnt = reinterpret_cast<unsigned*>(base + p.ws_cnt_off);
    a.ws_ml = reinterpret_cast<float*>(base + p.ws_ml_off);
    a.ws_o = reinterpret_cast<float*>(base + p.ws_o_off);
  }
  return a;
}

}  // namespace mgqa

using namespace mgqa;

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point (attn_fwd_noalloc): the split
// partials and arrival counters live in this file-scope device array instead
// of a caller or library allocation.  Each GPU the library runs on holds its
// own copy until the process ends.  In host code `scratch` is only a handle
// for the runtime: the device address of a GPU's copy comes from
// hipGetSymbolAddress with that GPU current, looked up once per device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[MGQA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
int g_scratch_err[kMaxDevices];

// Device address of the current GPU's scratch; on first use on a device its
// counter block is cleared on `stream` (the kernels leave the counters at zero
// after every completed call, so later calls need no clearing).
int scratch_for_current_device(void** out, void* stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MGQA_ERR_HIP;
  std::call_once(g_scratch_once[dev], [dev, stream] {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      g_scratch_err[dev] = MGQA_ERR_HIP;
      return;
    }
    if (launch_zero(ptr, kMaxCounters, stream) != hipSuccess) {
      g_scratch_err[dev] = MGQA_ERR_HIP;
      return;
    }
    g_scratch_ptr[dev] = ptr;
  });
  if (g_scratch_err[dev] != MGQA_OK) return g_scratch_err[dev];
  *out = g_scratch_ptr[dev];
  return MGQA_OK;
}
}  // namespace

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

extern "C" {

int attn_version(void) { return 104; }

const char* attn_error_string(int code) {
  switch (code) {
    case MGQA_OK: return "success";
    case MGQA_ERR_NULL: return "a required pointer is NULL";
    case MGQA_ERR_SHAPE: return "bad shape: sizes must be > 0, Hq a multiple of Hkv, Hq/Hkv <= 16";
    case MGQA_ERR_HEAD_DIM: return "unsupported head size: d must be a multiple of 8 and <= 128";
    case MGQA_ERR_MASK:
      return "bad mask: causal must be 0/1, window >= 0, and Lq <= Lkv when a causal mask or window is set";
    case MGQA_ERR_SOFTCAP: return "bad softcap: must be finite and >= 0";
    case MGQA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case MGQA_ERR_WORKSPACE: return "workspace missing or smaller than attn_workspace_bytes()";
    case MGQA_ERR_HIP: return "HIP runtime error or kernel launch failure";
    case MGQA_ERR_DTYPE: return "dtype must be MGQA_BF16 (0) or MGQA_FP16 (1)";
    case MGQA_ERR_RANGE: return "a size or position out of range (indexing limit, cache length, ring start, append position)";
    case MGQA_ERR_UNSUPPORTED: return "unsupported combination: a ring-buffer cache needs the decode path (Hq/Hkv * Lq <= 16)";
    default: return "unknown error code";
  }
}

int attn_plan(int B, int Hq, int Hkv, int Lq, int Lkv, int d, int causal, int window,
              float softcap, int dtype, long long info[12]) {
  if (!info) return MGQA_ERR_NULL;
  Plan p;
  const int err = make_plan(B, Hq, Hkv, Lq, Lkv, d, causal, window, softcap, dtype, &p);
  if (err) return err;
  info[0] = p.path;
  info[1] = p.workgroups;
  info[2] = p.rows_per_wg;
  info[3] = p.nsplit;
  info[4] = p.keys_per_tile;
  info[5] = p.qk_pad;
  info[6] = p.dv * 16;
  info[7] = (long long)p.ws_bytes;
  info[8] = p.ncol > 0 ? p.ncol : 1;
  const bool items = p.path == kPathPrefill && d == 128;
  info[9] = items ? p.pf_pairs : 0;
  info[10] = items ? p.pf_ramp : 0;
  info[11] = items ? p.pf_full : 0;
  return MGQA_OK;
}

size_t attn_workspace_bytes(int B, int Hq, int Hkv, int Lq, int Lkv, int d, int causal,
                            int window) {
  Plan p;
  if (make_plan(B, Hq, Hkv, Lq, Lkv, d, causal, window, 0.f, MGQA_BF16, &p)) return 0;
  return p.ws_bytes;
}

int attn_fwd_ex(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv,
                int Lq, int Lkv, int d, int causal, int window, float softcap, int dtype,
                void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !out) return MGQA_ERR_NULL;
  Plan p;
  const int err = make_plan(B, Hq, Hkv, Lq, Lkv, d, causal, window, softcap, dtype, &p);
  if (err) return err;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return MGQA_ERR_ALIGN;
  if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes)) return MGQA_ERR_WORKSPACE;
  if (p.ws_bytes > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u)) return MGQA_ERR_ALIGN;
  const KernelArgs a = make_args(p, q, k, v, out, Hq, Hkv, Lq, Lkv, d, causal, window, softcap,
                                 p.ws_bytes ? workspace : nullptr);
  if (launch(p, a, dtype, softcap > 0.f, stream) != hipSuccess) return MGQA_ERR_HIP;
  return MGQA_OK;
}

int attn_fwd_cache(const void* q, const void* k_cache, const void* v_cache, void* out, int B,
                   int Hq, int Hkv, int Lq, int S, int length, int ring_start, int d, int causal,
                   int window, float softcap, int dtype, void* workspace, size_t workspace_bytes,
                   void* stream) {
  if (!q || !k_cache || !v_cache || !out) return MGQA_ERR_NULL;
  if (S <= 0 || length <= 0) return MGQA_ERR_SHAPE;
  if (length > S) return MGQA_ERR_RANGE;
  if (ring_start < -1 || ring_start >= S) return MGQA_ERR_RANGE;
  if ((long long)S * d > kMaxUnitElems) return MGQA_ERR_RANGE;
  Plan p;
  const int err = make_plan(B, Hq, Hkv, Lq, length, d, causal, window, softcap, dtype, &p);
  if (err) return err;
  if (ring_start >= 0 && (p.path != kPathSplit || p.n_pos_blk != 1 || p.nqb != 1))
    return MGQA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return MGQA_ERR_ALIGN;
  if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes)) return MGQA_ERR_WORKSPACE;
  if (p.ws_bytes > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u)) return MGQA_ERR_ALIGN;
  KernelArgs a = make_args(p, q, k_cache, v_cache, out, Hq, Hkv, Lq, length, d, causal, window,
                           softcap, p.ws_bytes ? workspace : nullptr);
  a.kv_stride = (long long)S * d;
  a.ring_start = ring_start;
  a.ring_slots = S;
  if (launch(p, a, dtype, softcap > 0.f, stream) != hipSuccess) return MGQA_ERR_HIP;
  return MGQA_OK;
}

int attn_fwd_cache_append(const void* q, void* k_cache, void* v_cache, const float* new_k,
                          const float* new_v, void* out, int B, int Hq, int Hkv, int Lq, int S,
                          int position, int ring_start, int d, int causal, int window, float softcap,
                          int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_cache || !v_cache || !new_k || !new_v || !out) return MGQA_ERR_NULL;
  if (S <= 0 || Lq <= 0) return MGQA_ERR_SHAPE;
  if (position < 0 || Lq > S || position > S - Lq) return MGQA_ERR_RANGE;
  if (ring_start < -1 || ring_start >= S) return MGQA_ERR_RANGE;
  if ((long long)S * d > kMaxUnitElems) return MGQA_ERR_RANGE;
  const int length = position + Lq;
  Plan p;
  const int err = make_plan(B, Hq, Hkv, Lq, length, d, causal, window, softcap, dtype, &p);
  if (err) return err;
  if (ring_start >= 0 && (p.path != kPathSplit || p.n_pos_blk != 1 || p.nqb != 1))
    return MGQA_ERR_UNSUPPORTED;
  if ((long long)B * Hkv * Lq * d >= (1LL << 31)) return MGQA_ERR_RANGE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      !aligned16(new_k) || !aligned16(new_v))
    return MGQA_ERR_ALIGN;
  if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes)) return MGQA_ERR_WORKSPACE;
  if (p.ws_bytes > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u)) return MGQA_ERR_ALIGN;
  KernelArgs a = make_args(p, q, k_cache, v_cache, out, Hq, Hkv, Lq, length, d, causal, window,
                           softcap, p.ws_bytes ? workspace : nullptr);
  a.kv_stride = (long long)S * d;
  a.ring_start = ring_start;
  a.ring_slots = S;
  if (p.path == kPathSplit) {
    // One launch: the split-KV kernel takes the new keys from the float32
    // rows and writes them to the caches itself.
    a.app_k = new_k;
    a.app_v = new_v;
    a.app_pos = position;
    a.app_len = Lq;
  } else if (launch_append(k_cache, v_cache, new_k, new_v, B, S, Hkv, d, Lq, position, dtype, 1, nullptr,
                           stream) != hipSuccess) {
    return MGQA_ERR_HIP;
  }
  if (launch(p, a, dtype, softcap > 0.f, stream) != hipSuccess) return MGQA_ERR_HIP;
  return MGQA_OK;
}

int kv_cache_append(void* k_cache, void* v_cache, const float* new_k, const float* new_v, int B,
                    int S, int H, int D, int L, int position, int cache_dtype, int layout,
                    int* length_out, void* stream) {
  if (!k_cache || !v_cache || !new_k || !new_v) return MGQA_ERR_NULL;
  if (B <= 0 || S <= 0 || H <= 0 || D <= 0 || L <= 0) return MGQA_ERR_SHAPE;
  if (cache_dtype != MGQA_BF16 && cache_dtype != MGQA_FP16 && cache_dtype != MGQA_F32)
    return MGQA_ERR_DTYPE;
  if (layout != 0 && layout != 1) return MGQA_ERR_SHAPE;
  if (position < 0 || L > S || position > S - L) return MGQA_ERR_RANGE;
  if ((long long)B * S * H * D >= (1LL << 40) || (long long)B * L * H * D >= (1LL << 31))
    return MGQA_ERR_RANGE;
  if (launch_append(k_cache, v_cache, new_k, new_v, B, S, H, D, L, position, cache_dtype, layout,
                    length_out, stream) != hipSuccess)
    return MGQA_ERR_HIP;
  return MGQA_OK;
}

int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv,
                     int Lq, int Lkv, int d, int causal, int window, float softcap, int dtype,
                     void* stream) {
  if (!q || !k || !v || !out) return MGQA_ERR_NULL;
  Plan p;
  const int err = make_plan(B, Hq, Hkv, Lq, Lkv, d, causal, window, softcap, dtype, &p);
  if (err) return err;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return MGQA_ERR_ALIGN;
  if (p.ws_bytes > MGQA_NOALLOC_SCRATCH_BYTES) return MGQA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (p.ws_bytes > 0) {
    const int e = scratch_for_current_device(&ws, stream);
    if (e != MGQA_OK) return e;
  }
  const KernelArgs a = make_args(p, q, k, v, out, Hq, Hkv, Lq, Lkv, d, causal, window, softcap, ws);
  if (launch(p, a, dtype, softcap > 0.f, stream) != hipSuccess) return MGQA_ERR_HIP;
  return MGQA_OK;
}

int attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv,
             int Lq, int Lkv, int d, int causal, int window, float softcap, void* stream) {
  if (!q || !k || !v || !out) return MGQA_ERR_NULL;
  Plan p;
  const int err = make_plan(B, Hq, Hkv, Lq, Lkv, d, causal, window, softcap, MGQA_BF16, &p);
  if (err) return err;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return MGQA_ERR_ALIGN;
  if (p.ws_bytes == 0)
    return attn_fwd_ex(q, k, v, out, B, Hq, Hkv, Lq, Lkv, d, causal, window, softcap, MGQA_BF16,
                       nullptr, 0, stream);
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (hipMallocAsync(&ws, p.ws_bytes, st) != hipSuccess) return MGQA_ERR_HIP;
  // Only the counters must start at zero; the partials are always written first.
  int rc = MGQA_OK;
  if (launch_zero(ws, p.ws_ml_off / 4, stream) != hipSuccess) rc = MGQA_ERR_HIP;
  if (rc == MGQA_OK)
    rc = attn_fwd_ex(q, k, v, out, B, Hq, Hkv, Lq, Lkv, d, causal, window, softcap, MGQA_BF16, ws,
                     p.ws_bytes, stream);
  if (hipFreeAsync(ws, st) != hipSuccess && rc == MGQA_OK) rc = MGQA_ERR_HIP;
  return rc;
}

}  // extern "C"
