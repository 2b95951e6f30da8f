// extern "C" prefill entry points: validation of every host-visible argument,
// the device work list (built on the host, copied into the caller's
// workspace), the choice of dv split, and the launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <functional>
#include <numeric>
#include <string>
#include <unordered_set>
#include <vector>

#include "kda_hostutil.hpp"
#include "kda_internal.hpp"

using namespace kda_host;

namespace {

constexpr int kCUs = 256;  // MI355X compute units (one propagation workgroup per CU)

int64_t round8(int64_t x) { return (x + 7) / 8 * 8; }

// Chunks of one sequence: chunks never cross a checkpoint position.
int64_t seq_chunks(int32_t len, const int32_t* pos, int32_t npos, int32_t chunk) {
  int64_t c = 0;
  int32_t prev = 0;
  for (int32_t i = 0; i <= npos; ++i) {
    const int32_t next = i < npos ? pos[i] : len;
    c += (next - prev + chunk - 1) / chunk;
    prev = next;
  }
  return c;
}

// Chunks never cross a sequence end or a checkpoint, so a sequence of length
// L with m checkpoints has at most L / chunk + m + 1 of them.
int64_t max_chunks(int32_t n_seqs, int64_t total_tokens, int32_t chunk, int64_t n_ckpt) {
  return total_tokens / chunk + n_seqs + n_ckpt;
}

// Workspace: the int32 work list (a header of kHeaderInts words whose first
// is the decay-range flag, zero on entry; chains, sequence table,
// checkpoints, chunks, and room for a mixed-width workgroup list of up to
// eight entries per chain), then (256-byte aligned) one record per
// (chunk, head) (UnitLayout: T diag(beta), lower(A_qk) and the chunk's scaled
// operands, in the operand precision: bf16 for bf16 inputs, fp32 for fp32).
constexpr int64_t kHeaderInts = 64;
size_t work_ints(int32_t n_seqs, int32_t H, int64_t n_ckpt, int64_t n_chunks) {
  return static_cast<size_t>(kHeaderInts + 2 * round8(static_cast<int64_t>(n_seqs) * H) + 6 * n_seqs +
                             2 * n_ckpt + 2 * n_chunks + 8 * round8(static_cast<int64_t>(n_seqs) * H));
}

// Per-sequence tile widths: nw widths ws[0] > ws[1] > ... (columns per
// workgroup), with per-chunk times tw[j] measured with every CU busy
// (decreasing with the width) and mult[j] workgroups per head.  Each sequence
// takes the widest width whose chain fits a target time; the target is the
// one that balances the longest chain against the total work over the CUs.
// The candidate targets are the chains' own times at each width; with the
// chunk counts sorted and summed once, each candidate costs nw - 1 binary
// searches, so the choice is O(n log n) in the number of sequences.  Returns
// the predicted time (us) and fills width[s].
double choose_widths(const std::vector<int64_t>& chunks, int32_t H, const int* ws, const double* tw,
                     const double* mult, int nw, std::vector<int>& width, double fixed_work = 0,
                     double fixed_longest = 0) {
  const size_t n = chunks.size();
  std::vector<int64_t> c(chunks);
  std::sort(c.begin(), c.end());
  std::vector<double> pre(n + 1, 0.0);
  for (size_t i = 0; i < n; ++i) pre[i + 1] = pre[i] + static_cast<double>(c[i]);
  // Sequences [0, fits(j, T)) of the sorted list fit the target T at width j.
  auto fits = [&](int j, double T) {
    return static_cast<size_t>(std::partition_point(c.begin(), c.end(), [&](int64_t x) {
                                 return static_cast<double>(x) * tw[j] <= T;
                               }) - c.begin());
  };
  // (fixed_work, fixed_longest: chains whose width is not chosen here)
  auto cost_at = [&](double T) {
    double work = fixed_work, longest = fixed_longest;
    size_t prev = 0;
    for (int j = 0; j < nw; ++j) {
      const size_t e = j + 1 < nw ? std::max(prev, fits(j, T)) : n;  // group j: [prev, e)
      work += H * mult[j] * tw[j] * (pre[e] - pre[prev]);
      if (e > prev) longest = std::max(longest, static_cast<double>(c[e - 1]) * tw[j]);
      prev = e;
    }
    return std::max(longest, work / kCUs);
  };
  double best = 0, best_T = 0;
  if (n == 0) best = std::max(fixed_longest, fixed_work / kCUs);
  for (size_t i = 0; i < n; ++i) {
    if (i > 0 && c[i] == c[i - 1]) continue;
    for (int j = 0; j < nw; ++j) {
      const double T = static_cast<double>(c[i]) * tw[j];
      const double cost = cost_at(T);
      // On a tie the larger target wins: wider tiles, less total work.
      if (best == 0 || cost < best * (1 - 1e-12) || (cost <= best * (1 + 1e-12) && T > best_T)) {
        best = std::min(best == 0 ? cost : best, cost);
        best_T = T;
      }
    }
  }
  width.assign(n, ws[nw - 1]);
  for (size_t s = 0; s < n; ++s)
    for (int j = 0; j < nw; ++j)
      if (static_cast<double>(chunks[s]) * tw[j] <= best_T) {
        width[s] = ws[j];
        break;
      }
  return best;
}

// The fused kernel's per-chunk times (us, 32-token chunks) at 128, 64, 32
// and 16 columns per workgroup, measured on MI355X (one workgroup per CU).
constexpr int kFusedW[4] = {128, 64, 32, 16};
constexpr double kFusedT[4] = {2.66, 2.27, 2.01, 2.14};
bool fused_path(kda_dtype in_dtype, int32_t dk, int32_t chunk) {
  return in_dtype == KDA_BF16 && chunk == 32 && dk == 128;
}

// Segments of long sequences in the fused launch (context parallelism on one
// GPU; the "Serve 模块交互式演示" page's §1.7 and §7.2 reduce a segment to a
// fixed-size map of its start state and compose the maps).  A split
// sequence's first segment runs from s0 as usual; each later segment runs
// twice beside it, from the zero state (kind 1) and from the identity with v
// taken as zero (kind 2: its linear part, one 128-column tile); workgroups at
// the launch's tail then chain the maps into the segments' start states and
// correct the later segments' outputs and checkpoints (kda_fused.hip,
// fused_tail; kda_cp.hpp).  It pays where the longest chain bounds the call:
// each segment's chain is shorter, for the identity chains' work and the
// correction's traffic.
constexpr int kMaxExtraSegs = 8;          // later segments per call (bounds the workspace)
constexpr int32_t kTailBlock = 192;       // rows of a tail item's block (16 per wave of the fused kernel)
constexpr int32_t kTailTokens = 1536;     // rows per tail item of the correction, at most (8 blocks)
constexpr int kMinSegChunks = 16;         // chunks per segment, at least
constexpr double kTailBytesPerUs = 5.0e6;    // the tail items' cost, bytes per us of the call
constexpr double kTailStateUs = 20.0;        // a tail item forming a start state (they run in turn)
constexpr double kChainUs = 15.0;            // a chain's fixed cost (its prologue), us
constexpr int64_t kMaxSimWgs = 200000;       // workgroups the plan's list scheduling models at most

// One chain set of the fused launch: a whole sequence, or a segment.
struct Entry {
  int32_t seq = 0, kind = 0, seg = 0;  // kind 0: a whole sequence or a first segment, 1: from zero, 2: from the identity
  int32_t lo = 0, hi = 0;              // tokens [lo, hi) from the sequence's first
  int32_t ck0 = 0, ck1 = 0;            // its checkpoints: the sequence's entries [ck0, ck1), positions in (lo, hi]
  int64_t chunks = 0;
  int width = 0;                       // columns per workgroup
};

// Cut points of len tokens into n segments, on multiples of the chunk
// (len >= n * kMinSegChunks * chunk keeps them increasing and inside).
std::vector<int32_t> seg_bounds(int32_t len, int n, int32_t chunk) {
  std::vector<int32_t> b(n + 1, 0);
  b[n] = len;
  for (int i = 1; i < n; ++i) {
    const int64_t t = static_cast<int64_t>(len) * i / n;
    b[i] = static_cast<int32_t>((t + chunk / 2) / chunk * chunk);
  }
  return b;
}

// The entries of sequence s (len tokens, checkpoint positions pos[0..npos))
// in n segments.
void seq_entries(int32_t s, int32_t len, const int32_t* pos, int32_t npos, int n, int32_t chunk,
                 std::vector<Entry>& out) {
  const std::vector<int32_t> b = seg_bounds(len, n, chunk);
  int32_t c = 0;
  std::vector<int32_t> lp;
  for (int k = 0; k < n; ++k) {
    int32_t c1 = c;
    lp.clear();
    while (c1 < npos && pos[c1] <= b[k + 1]) lp.push_back(pos[c1++] - b[k]);
    Entry e;
    e.seq = s;
    e.seg = k;
    e.lo = b[k];
    e.hi = b[k + 1];
    e.ck0 = c;
    e.ck1 = c1;
    e.chunks = seq_chunks(b[k + 1] - b[k], lp.data(), c1 - c, chunk);
    e.kind = k == 0 ? 0 : 1;
    out.push_back(e);
    if (k > 0) {
      e.kind = 2;
      out.push_back(e);
    }
    c = c1;
  }
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }
size_t tile_bytes(int64_t n_chunks, int32_t H, int32_t chunk, int32_t dk, size_t es) {
  return static_cast<size_t>(n_chunks) * H * kda::UnitLayout(chunk, dk, static_cast<int>(es)).bytes;
}

// dv columns per workgroup: 16, 32 or 64 (a 128-column tile's buffers do not
// fit in LDS).
// Slab-format records and the column-slab propagation kernel: bf16 inputs,
// chunk 64, dk a multiple of 32.
bool slab_path(int32_t dk, bool bf16, int32_t chunk) { return bf16 && chunk == 64 && dk % 32 == 0; }

bool valid_tile(int32_t dv, int32_t split, bool slab) {
  if (split != 1 && split != 2 && split != 4 && split != 8) return false;
  if (dv % split) return false;
  const int t = dv / split;
  return t == 16 || t == 32 || t == 64 || (slab && t == 128);
}

// Pick the dv split from a per-chunk cost model (MFMA tile counts): key-side
// work (Gram products, T) is repeated by every split, value-side work scales
// with the tile width; the chip time is the larger of the total work over the
// CUs and the longest chain.
int choose_split(int32_t dk, int32_t dv, bool bf16, int64_t total_chunks, int64_t longest) {
  int best = 0;
  double best_t = 0;
  for (int split : {1, 2, 4, 8}) {
    if (!valid_tile(dv, split, false)) continue;
    const double tile = static_cast<double>(dv) / split;
    const double cost = 1.5 * dk + (3.0 * dk / 8 + 12.0) * tile / 16.0;
    const double t = std::max(static_cast<double>(total_chunks) * split * cost / kCUs,
                              static_cast<double>(longest) * cost);
    if (best == 0 || t < best_t * 0.999) {
      best = split;
      best_t = t;
    }
  }
  return best;
}

// The column-slab kernel's split: a workgroup per (chain, tile) holds a CU
// (its LDS), and a chunk costs it about t(tile) whatever else runs, set by
// how fast one CU streams the chunk's record from HBM and by its waves'
// serial work (measured on MI355X: about 3.0, 2.4, 2.0 and 1.95 us per
// chunk at 128, 64, 32 and 16 columns).  The call takes about the larger of
// the longest chain and the total work over the CUs.
int choose_split_slab(int32_t dv, int64_t total_chunks, int64_t longest) {
  int best = 0;
  double best_t = 0;
  for (int split : {1, 2, 4, 8}) {
    if (!valid_tile(dv, split, true)) continue;
    const int tile = dv / split;
    const double t = tile == 128 ? 3.0 : tile == 64 ? 2.4 : tile == 32 ? 2.0 : 1.95;
    const double cost = std::max(static_cast<double>(total_chunks) * split * t / kCUs,
                                 static_cast<double>(longest) * t);
    if (best == 0 || cost < best_t * 0.999) {
      best = split;
      best_t = cost;
    }
  }
  return best;
}

// What a call will launch: validated shapes and offsets, chunk counts, the
// dv split and (mixed launch) a tile width per sequence.
struct Plan {
  int64_t n_chunks = 0, longest = 0;
  int split = 0, a_split = 0;
  bool slab = false, mixed = false, fused = false;
  std::vector<int> width;  // columns per workgroup, per sequence (a split one: its first segment's)
  // The fused launch: its chain sets, and the segments per sequence (cp: any
  // sequence in more than one).
  std::vector<Entry> ent;
  std::vector<int> nseg;
  bool cp = false;
};

// Validates everything the plan depends on (dtype, sizes, cu_seqlens,
// checkpoint offsets and positions; not buffers or slots) and makes the plan.
int make_plan(kda_dtype in_dtype, int32_t H, int32_t dk, int32_t dv, int32_t chunk, const int32_t* cu,
              int32_t n_seqs, const int32_t* ck_cu, const int32_t* ck_pos, int64_t n_ckpt, int32_t dv_split,
              bool summary, Plan& pl, bool allow_cp = true) {
  if (!valid_dtype(in_dtype)) return fail(KDA_EINVAL, "in_dtype %d", static_cast<int>(in_dtype));
  if (n_seqs < 0 || H <= 0 || n_ckpt < 0)
    return fail(KDA_EINVAL, "n_seqs=%d H=%d n_ckpt=%lld", n_seqs, H, static_cast<long long>(n_ckpt));
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(KDA_EUNSUPPORTED, "dk=%d dv=%d (supported: 16, 32, 64, 128)", dk, dv);
  if (chunk < 16 || chunk > KDA_MAX_CHUNK || chunk % 16)
    return fail(KDA_EUNSUPPORTED, "chunk=%d (a multiple of 16 up to %d)", chunk, KDA_MAX_CHUNK);
  if (in_dtype == KDA_F32 && chunk > 32)
    return fail(KDA_EUNSUPPORTED, "chunk=%d: fp32 inputs take chunks of at most 32 rows", chunk);
  const int64_t hkv = static_cast<int64_t>(H) * dk * dv;
  if (hkv >= (int64_t{1} << 31)) return fail(KDA_EUNSUPPORTED, "H*dk*dv must be below 2^31");
  const int64_t hkk = static_cast<int64_t>(H) * dk * dk;
  if (summary && hkk >= (int64_t{1} << 31)) return fail(KDA_EUNSUPPORTED, "H*dk*dk must be below 2^31");
  // The kernel addresses one chunk's rows with 32-bit byte offsets.
  if (static_cast<int64_t>(H) * std::max(dk, dv) > (int64_t{1} << 24))
    return fail(KDA_EUNSUPPORTED, "H*max(dk, dv) must be at most 2^24");
  if (n_seqs > 0) {
    if (!cu) return fail(KDA_EINVAL, "cu_seqlens is null");
    if (cu[0] != 0) return fail(KDA_EINVAL, "cu_seqlens[0] = %d, must be 0", cu[0]);
    for (int32_t i = 0; i < n_seqs; ++i)
      if (cu[i + 1] < cu[i]) return fail(KDA_EINVAL, "cu_seqlens decreases at %d", i);
  }

  // Checkpoints: the offsets first (all of them, so that no position is read
  // through an offset a later entry would have refused), then the positions.
  if (n_ckpt > 0 && (!ck_cu || !ck_pos)) return fail(KDA_EINVAL, "checkpoints need ckpt_cu and ckpt_pos");
  if (ck_cu && n_seqs > 0) {
    if (ck_cu[0] != 0) return fail(KDA_EINVAL, "ckpt_cu must start at 0");
    for (int32_t i = 0; i < n_seqs; ++i)
      if (ck_cu[i + 1] < ck_cu[i] || ck_cu[i + 1] > n_ckpt)
        return fail(KDA_EINVAL, "ckpt_cu must be non-decreasing and at most n_ckpt (entry %d)", i + 1);
    if (ck_cu[n_seqs] != n_ckpt) return fail(KDA_EINVAL, "ckpt_cu must end at n_ckpt");
    for (int32_t i = 0; i < n_seqs; ++i) {
      const int32_t len = cu[i + 1] - cu[i];
      for (int32_t c = ck_cu[i]; c < ck_cu[i + 1]; ++c) {
        if (ck_pos[c] < 1 || ck_pos[c] > len)
          return fail(KDA_EINVAL, "checkpoint %d of sequence %d at %d outside 1..%d", c - ck_cu[i], i,
                      ck_pos[c], len);
        if (c > ck_cu[i] && ck_pos[c] <= ck_pos[c - 1])
          return fail(KDA_EINVAL, "checkpoints of sequence %d not strictly increasing", i);
      }
    }
  } else if (n_ckpt != 0) {
    return fail(KDA_EINVAL, "n_ckpt > 0 without ckpt_cu");
  }

  // Chunks and split.
  pl = Plan{};
  const int64_t n_chains = round8(static_cast<int64_t>(n_seqs) * H);
  for (int32_t i = 0; i < n_seqs; ++i) {
    const int32_t len = cu[i + 1] - cu[i];
    const int32_t c0 = ck_cu ? ck_cu[i] : 0, c1 = ck_cu ? ck_cu[i + 1] : 0;
    const int64_t c = seq_chunks(len, ck_pos ? ck_pos + c0 : nullptr, c1 - c0, chunk);
    pl.n_chunks += c;
    pl.longest = std::max(pl.longest, c);
  }
  if (pl.n_chunks * H >= (int64_t{1} << 31)) return fail(KDA_EUNSUPPORTED, "too many (chunk, head) pairs");
  const bool bf16 = in_dtype == KDA_BF16;
  // The fused kernel (bf16, chunk 32, dk 128): a tile width per sequence,
  // 16 to 128 columns, from its cost model, or one width dv / dv_split; long
  // sequences possibly in segments (dv_split 0: where the model predicts it
  // faster; -n, 2 <= n <= 8: every sequence of at least n * kMinSegChunks
  // chunks in n segments, as far as kMaxExtraSegs allows).
  if (fused_path(in_dtype, dk, chunk) && !summary) {
    pl.fused = true;
    int fixed_w = 0;
    if (dv_split > 0) {
      fixed_w = dv % dv_split ? 0 : dv / dv_split;
      if (fixed_w != 16 && fixed_w != 32 && fixed_w != 64 && fixed_w != 128)
        return fail(KDA_EUNSUPPORTED, "dv_split=%d with dv=%d (dv/split must be 16, 32, 64 or 128)", dv_split, dv);
      pl.split = dv_split;
    } else if (dv_split < -kMaxExtraSegs) {
      return fail(KDA_EUNSUPPORTED, "dv_split=%d", dv_split);
    }
    std::vector<int64_t> sc(n_seqs);
    for (int32_t i = 0; i < n_seqs; ++i) {
      const int32_t c0 = ck_cu ? ck_cu[i] : 0, c1 = ck_cu ? ck_cu[i + 1] : 0;
      sc[i] = seq_chunks(cu[i + 1] - cu[i], ck_pos ? ck_pos + c0 : nullptr, c1 - c0, chunk);
    }
    int ws[4], nw = 0;
    double tw[4], mult[4];
    for (int j = 0; j < 4; ++j)
      if (kFusedW[j] <= dv) {
        ws[nw] = kFusedW[j];
        tw[nw] = kFusedT[j];
        mult[nw] = static_cast<double>(dv) / kFusedW[j];
        ++nw;
      }
    auto entries = [&](const std::vector<int>& ns) {
      std::vector<Entry> ent;
      for (int32_t i = 0; i < n_seqs; ++i) {
        const int32_t c0 = ck_cu ? ck_cu[i] : 0, c1 = ck_cu ? ck_cu[i + 1] : 0;
        seq_entries(i, cu[i + 1] - cu[i], ck_pos ? ck_pos + c0 : nullptr, c1 - c0, ns[i], chunk, ent);
      }
      return ent;
    };
    // Widths of the entries (identity chains: 128 columns) and the predicted
    // time, the correction included.
    // (the correction, the launch's tail items, lengthens the call by about
    // their bytes at kTailBytesPerUs, and by the start states formed in turn)
    auto assign = [&](std::vector<Entry>& ent, const std::vector<int>& ns) {
      std::vector<int64_t> ch;
      double fixed_work = 0, fixed_longest = 0, tail = 0, chain_states = 0;
      for (const Entry& e : ent) {
        if (e.kind == 2) {
          fixed_work += static_cast<double>(H) * kFusedT[0] * static_cast<double>(e.chunks);
          fixed_longest = std::max(fixed_longest, kFusedT[0] * static_cast<double>(e.chunks));
          tail += static_cast<double>(e.hi - e.lo) * H * (2.0 * dk + 4.0 * dv) / kTailBytesPerUs;
          chain_states = std::max(chain_states, kTailStateUs * (ns[e.seq] - 2));
        } else {
          ch.push_back(e.chunks);
        }
      }
      std::vector<int> w;
      double t;
      if (fixed_w) {
        w.assign(ch.size(), fixed_w);
        double work = fixed_work, longest = fixed_longest;
        int j = 0;
        while (ws[j] != fixed_w) ++j;
        for (int64_t c : ch) {
          work += H * mult[j] * tw[j] * static_cast<double>(c);
          longest = std::max(longest, tw[j] * static_cast<double>(c));
        }
        t = std::max(longest, work / kCUs);
      } else {
        t = ch.empty() ? std::max(fixed_longest, fixed_work / kCUs)
                       : choose_widths(ch, H, ws, tw, mult, nw, w, fixed_work, fixed_longest);
      }
      size_t j = 0;
      for (Entry& e : ent) e.width = e.kind == 2 ? 128 : w[j++];
      // The chains' workgroups, longest first, list-scheduled on the CUs: a
      // few hundred equal chains fill the CUs in whole rounds, which the
      // work over the CUs does not show.
      std::vector<double> d;
      for (const Entry& e : ent) {
        const int k = e.width == 128 ? 0 : e.width == 64 ? 1 : e.width == 32 ? 2 : 3;
        const int tiles = e.kind == 2 ? 1 : dv / e.width;
        if (static_cast<int64_t>(d.size()) + static_cast<int64_t>(tiles) * H > kMaxSimWgs) {
          d.clear();
          break;
        }
        d.insert(d.end(), static_cast<size_t>(tiles) * H, kFusedT[k] * static_cast<double>(e.chunks) + kChainUs);
      }
      if (!d.empty()) {
        std::sort(d.begin(), d.end(), std::greater<double>());
        std::vector<double> cus(kCUs, 0.0);
        double span = 0;
        for (double x : d) {
          std::pop_heap(cus.begin(), cus.end(), std::greater<double>());
          cus.back() += x;
          span = std::max(span, cus.back());
          std::push_heap(cus.begin(), cus.end(), std::greater<double>());
        }
        t = std::max(t, span);
      }
      return t + tail + chain_states;
    };
    pl.nseg.assign(n_seqs, 1);
    const bool cp_ok = allow_cp && dv == dk && dv == 128 && n_seqs > 0;
    auto min_len = [&](int n) { return static_cast<int64_t>(n) * kMinSegChunks * chunk; };
    if (cp_ok && dv_split <= -2) {
      int extra = 0;
      for (int32_t i = 0; i < n_seqs; ++i)
        if (cu[i + 1] - cu[i] >= min_len(-dv_split) && extra + (-dv_split - 1) <= kMaxExtraSegs) {
          pl.nseg[i] = -dv_split;
          extra += -dv_split - 1;
        }
    } else if (cp_ok && dv_split == 0) {
      // Greedy: give the sequence with the longest segments one more segment
      // while the model predicts at least 2 % less time.
      std::vector<Entry> ent = entries(pl.nseg);
      double best = assign(ent, pl.nseg);
      for (int extra = 0; extra < kMaxExtraSegs; ++extra) {
        int32_t top = -1;
        for (int32_t i = 0; i < n_seqs; ++i)
          if (cu[i + 1] - cu[i] >= min_len(pl.nseg[i] + 1) &&
              (top < 0 || sc[i] * pl.nseg[top] > sc[top] * pl.nseg[i]))
            top = i;
        if (top < 0) break;
        ++pl.nseg[top];
        ent = entries(pl.nseg);
        const double t = assign(ent, pl.nseg);
        if (t < 0.98 * best) {
          best = t;
        } else {
          --pl.nseg[top];
          break;
        }
      }
    }
    pl.ent = entries(pl.nseg);
    assign(pl.ent, pl.nseg);
    pl.cp = std::any_of(pl.nseg.begin(), pl.nseg.end(), [](int n) { return n > 1; });
    pl.width.assign(n_seqs, 0);
    for (const Entry& e : pl.ent)
      if (e.kind == 0) pl.width[e.seq] = e.width;
    if (round8(static_cast<int64_t>(pl.ent.size()) * H) >= (int64_t{1} << 23))
      return fail(KDA_EUNSUPPORTED, "too many chains");
    pl.mixed = dv_split <= 0;
    return KDA_OK;
  }
  pl.slab = slab_path(dk, bf16, chunk);
  // -1: a width per sequence (mixed launch), where the slab kernel runs at dv = 128.
  const bool force_mixed = dv_split == -1;
  if (force_mixed && (!pl.slab || dv != 128 || summary))
    return fail(KDA_EUNSUPPORTED, "dv_split=-1 needs bf16 inputs, chunk 64, dk a multiple of 32 and dv = 128");
  pl.split = dv_split;
  if (pl.split == 0 || force_mixed)
    pl.split = pl.slab ? choose_split_slab(dv, pl.n_chunks * H, pl.longest)
                       : choose_split(dk, dv, bf16, pl.n_chunks * H, pl.longest);
  if (!valid_tile(dv, pl.split, pl.slab))
    return fail(KDA_EUNSUPPORTED, "dv_split=%d with dv=%d (dv/split must be 16, 32 or 64%s)", dv_split, dv,
                pl.slab ? ", or 128" : "");
  if (n_chains * pl.split >= (int64_t{1} << 31)) return fail(KDA_EUNSUPPORTED, "too many chains");
  // The linear part A of a summary propagates dk identity columns.
  pl.a_split = !summary ? 0 : pl.slab ? choose_split_slab(dk, pl.n_chunks * H, pl.longest)
                                      : choose_split(dk, dk, bf16, pl.n_chunks * H, pl.longest);
  pl.width.assign(n_seqs, dv / pl.split);

  // Mixed tile widths: at dv = 128 on the slab path (prefill, automatic
  // split), when the per-sequence widths predict a time 3 % or more below
  // the single width's, the propagation runs one workgroup list with a width
  // per sequence (kda_prefill_slab.hpp, slab_mixed_kernel).  Its entries
  // pack the chain index above 8 bits, so it needs fewer than 2^23 chains.
  if (pl.slab && !summary && dv == 128 && (dv_split == 0 || force_mixed) && n_seqs > 0 &&
      n_chains < (int64_t{1} << 23)) {
    std::vector<int64_t> sc(n_seqs);
    int64_t total = 0;
    for (int32_t i = 0; i < n_seqs; ++i) {
      const int32_t c0 = ck_cu ? ck_cu[i] : 0, c1 = ck_cu ? ck_cu[i + 1] : 0;
      sc[i] = seq_chunks(cu[i + 1] - cu[i], ck_pos ? ck_pos + c0 : nullptr, c1 - c0, chunk);
      total += sc[i];
    }
    std::vector<int> width;
    const int ws[3] = {128, 64, 32};
    const double tw[3] = {3.8, 2.5, 2.0}, mult[3] = {1, 2, 4};
    const double tm = choose_widths(sc, H, ws, tw, mult, 3, width);
    // The best single width by the same per-chunk times (16 columns: 1.95 us).
    double tu = 0;
    const int uw[4] = {16, 32, 64, 128};
    const double ut[4] = {1.95, 2.0, 2.5, 3.8};
    for (int j = 0; j < 4; ++j) {
      const double c = std::max(static_cast<double>(pl.longest) * ut[j],
                                static_cast<double>(total) * H * (128 / uw[j]) * ut[j] / kCUs);
      if (tu == 0 || c < tu) tu = c;
    }
    if (tm > 0 && (force_mixed || tm < 0.97 * tu)) {
      pl.mixed = true;
      pl.width = width;
    }
  }
  return KDA_OK;
}

// Names of the kernels a plan launches (for reports).
std::string plan_kernels(const Plan& pl, kda_dtype in_dtype, int32_t dk, int32_t dv, bool gate) {
  const char* t = in_dtype == KDA_BF16 ? "bf16" : "fp32";
  char buf[256];
  const std::string local = std::string("local_kernel<") + std::to_string(dk) + "," + t + (gate ? ",gated" : "") + ">";
  if (pl.fused) {
    int lo = 1 << 30, hi = 0;
    for (int w : pl.width) { lo = std::min(lo, w); hi = std::max(hi, w); }
    snprintf(buf, sizeof(buf), "fused_kernel<%d> (32-token chunks, records in LDS; %d to %d columns per workgroup)",
             dk, pl.width.empty() ? 0 : lo, hi);
    if (pl.cp) {
      int n_split = 0, n_seg = 0;
      for (int n : pl.nseg)
        if (n > 1) {
          ++n_split;
          n_seg += n;
        }
      const size_t len = strlen(buf);
      snprintf(buf + len, sizeof(buf) - len, "; %d sequence%s in %d segments", n_split, n_split == 1 ? "" : "s",
               n_seg);
    }
  } else if (pl.mixed)
    snprintf(buf, sizeof(buf), "%s + slab_mixed_kernel<%d> (a tile width per sequence)", local.c_str(), dk);
  else if (pl.slab)
    snprintf(buf, sizeof(buf), "%s + slab_kernel<%d> (%d-column tiles)", local.c_str(), dk, dv / pl.split);
  else
    snprintf(buf, sizeof(buf), "%s + prop_kernel<%d,%d,%s>", local.c_str(), dk, dv / pl.split, t);
  return buf;
}


// The fused launch's work list (copied into the workspace as one block of
// int32) and the buffers that split sequences need behind it.
struct FusedList {
  std::vector<int32_t> w;
  size_t chains = 0, seqinfo = 0, segx = 0, ck_pos = 0, ck_slot = 0, wgs = 0, titems = 0, tcnt = 0;
  int64_t n_chains = 0, n_wg = 0, n_cnt = 0;
  int64_t n_tstate = 0, n_xpool = 0, n_qrows = 0;  // states of H*dk*dv fp32; qhat rows of H*dk bf16
  bool items_fit = true;  // the tail items' indices fit their 23 bits of a workgroup entry
  size_t list_bytes() const { return align256(w.size() * 4); }
};

// Builds the list (ck_slot may be null when only the sizes are wanted).
FusedList fused_list(const Plan& pl, const int32_t* cu, const int32_t* ck_cu, const int32_t* ck_pos,
                     const int32_t* ck_slot, int32_t H, int32_t dv, bool want_final) {
  FusedList f;
  const std::vector<Entry>& ent = pl.ent;
  const int64_t n_ent = static_cast<int64_t>(ent.size());
  // Per split sequence in n segments: its tstate block (E1, the end state of
  // segment 0; A_j, B_j of segments 1..n-1; the start states S_j of segments
  // 2..n-1), and per segment j >= 1 and head a completion counter (cbase +
  // (j - 1) H + head): raised by the chains of segment j (from zero and from
  // the identity) and by what forms its start state (segment 0's chain for
  // j = 1, the tail item S_j = A_{j-1} S_{j-1} + B_{j-1} after), 0x10000 for
  // one that stopped at a decay out of range; cwant[s][j] counts them.
  std::vector<int64_t> tbase(pl.nseg.size(), -1);
  std::vector<int32_t> cbase(pl.nseg.size(), -1);
  std::vector<std::vector<int32_t>> cwant(pl.nseg.size());
  for (size_t s = 0; s < pl.nseg.size(); ++s)
    if (pl.nseg[s] > 1) {
      tbase[s] = f.n_tstate;
      cbase[s] = static_cast<int32_t>(f.n_cnt);
      f.n_tstate += 3 * pl.nseg[s] - 2;
      f.n_cnt += static_cast<int64_t>(pl.nseg[s] - 1) * H;
      cwant[s].assign(pl.nseg[s], 0);
      for (int j = 2; j < pl.nseg[s]; ++j) cwant[s][j] = 1;  // the tail item forming S_j
    }
  auto seg_of = [](const Entry& e) { return e.kind == 0 ? 1 : e.seg; };  // (the counter a chain raises)
  for (const Entry& e : ent)
    if (pl.nseg[e.seq] > 1) cwant[e.seq][seg_of(e)] += e.kind == 2 ? 1 : dv / e.width;
  // The later segments of split sequences, as the tail items need them.
  struct Later {
    int32_t seq, j, lo, len, qrow, ck0, ck1;
    int64_t xp;  // xpool index of its first checkpoint's B (X at + 1)
  };
  std::vector<Later> later;
  std::vector<int32_t> seqinfo(6 * n_ent), segx(pl.cp ? kda::kSegxInts * n_ent : 0), pos, slot;
  int64_t nc = 0;
  for (int64_t i = 0; i < n_ent; ++i) {
    const Entry& e = ent[i];
    const int32_t sq = e.seq, n = pl.nseg[sq], cb = ck_cu ? ck_cu[sq] : 0;
    int32_t* si = &seqinfo[6 * i];
    si[0] = cu[sq] + e.lo;
    si[1] = cu[sq] + e.hi;
    si[2] = static_cast<int32_t>(pos.size());
    for (int32_t c = e.ck0; c < e.ck1; ++c) {
      pos.push_back(ck_pos[cb + c] - e.lo);
      int32_t sl = 0;
      if (e.kind == 0) sl = ck_slot ? ck_slot[cb + c] : 0;
      else sl = static_cast<int32_t>(f.n_xpool + 2 * (c - e.ck0) + (e.kind == 2));
      slot.push_back(sl);
    }
    si[3] = static_cast<int32_t>(pos.size());
    si[4] = static_cast<int32_t>(nc);
    nc += e.chunks;
    si[5] = static_cast<int32_t>(nc);
    if (!pl.cp) continue;
    int32_t* sx = &segx[kda::kSegxInts * i];
    const int64_t b = tbase[sq];
    sx[4] = n > 1 ? cbase[sq] + (seg_of(e) - 1) * H : -1;
    if (n == 1) {
      sx[0] = sx[1] = sq;
    } else if (e.kind == 0) {  // the first segment: from s0, its end state is E1
      sx[0] = sq;
      sx[1] = static_cast<int32_t>(b);
      sx[2] = kda::kSegFinalTemp;
    } else if (e.kind == 1) {  // from zero: B of segment e.seg
      sx[1] = static_cast<int32_t>(b + (n - 1) + e.seg);
      sx[2] = kda::kSegZeroStart | kda::kSegFinalTemp | kda::kSegCkTemp;
    } else {  // from the identity: A of segment e.seg, outputs to qhat
      sx[1] = static_cast<int32_t>(b + e.seg);
      sx[3] = static_cast<int32_t>(f.n_qrows);
      later.push_back({sq, e.seg, cu[sq] + e.lo, e.hi - e.lo, static_cast<int32_t>(f.n_qrows), e.ck0, e.ck1, f.n_xpool});
      f.n_xpool += 2 * (e.ck1 - e.ck0);
      f.n_qrows += e.hi - e.lo;
    }
  }
  // Tail items (kTailInts each; see fused_tail): the start states S_j (j >= 2)
  // first, in order, then per segment and head its output rows, checkpoints
  // and (last segment) the sequence's final state.  An item waits for the
  // counter of its segment; an item forming S_j raises S_j's counter.
  std::vector<int32_t> titems;
  auto tstart = [&](const Later& g) {  // tstate index of the segment's start state
    const int64_t b = tbase[g.seq];
    return static_cast<int32_t>(g.j == 1 ? b : b + 2 * (pl.nseg[g.seq] - 1) + g.j);
  };
  auto cnt_of = [&](int32_t sq, int j, int32_t h) { return cbase[sq] + (j - 1) * H + h; };
  for (const Later& g : later) {
    const int32_t n = pl.nseg[g.seq];
    if (g.j + 1 >= n) continue;
    const int64_t b = tbase[g.seq];
    Later nx = g;
    nx.j = g.j + 1;
    for (int32_t h = 0; h < H; ++h)  // S_{j+1} = A_j S_j + B_j
      titems.insert(titems.end(), {1, 2, tstart(nx), static_cast<int32_t>(b + (n - 1) + g.j),
                                   static_cast<int32_t>(b + g.j), tstart(g), 1, h, cnt_of(g.seq, g.j, h),
                                   cwant[g.seq][g.j], cnt_of(g.seq, g.j + 1, h), 0});
  }
  // Rows per item: about two items per CU over all later segments' rows,
  // in whole blocks of the tail's 192 rows, at most kTailTokens.
  int64_t rows_total = 0;
  for (const Later& g : later) rows_total += static_cast<int64_t>(g.len) * H;
  const int32_t per_item = static_cast<int32_t>(std::min<int64_t>(
      kTailTokens, std::max<int64_t>(1, (rows_total / (2 * kCUs) + kTailBlock - 1) / kTailBlock) * kTailBlock));
  for (const Later& g : later) {
    const int32_t n = pl.nseg[g.seq], cb = ck_cu ? ck_cu[g.seq] : 0, sin = tstart(g);
    const int64_t b = tbase[g.seq];
    for (int32_t h = 0; h < H; ++h) {
      const int32_t cnt = cnt_of(g.seq, g.j, h), want = cwant[g.seq][g.j];
      for (int32_t t0 = 0; t0 < g.len; t0 += per_item)
        titems.insert(titems.end(), {0, g.lo, g.len, g.qrow, sin, h, t0, std::min(g.len, t0 + per_item), cnt,
                                     want, -1, 0});
      for (int32_t c = g.ck0; c < g.ck1; ++c)
        titems.insert(titems.end(), {1, 0, ck_slot ? ck_slot[cb + c] : 0, static_cast<int32_t>(g.xp + 2 * (c - g.ck0)),
                                     static_cast<int32_t>(g.xp + 2 * (c - g.ck0) + 1), sin, 0, h, cnt, want, -1, 0});
      if (want_final && g.j == n - 1)  // the final state A_{n-1} S_{n-1} + B_{n-1}
        titems.insert(titems.end(), {1, 1, g.seq, static_cast<int32_t>(b + (n - 1) + g.j),
                                     static_cast<int32_t>(b + g.j), sin, 1, h, cnt, want, -1, 0});
    }
  }
  // Chains: the entries' heads, the longest chain first, padded to whole
  // rounds of eight (one per XCD).
  std::vector<int64_t> order(n_ent);
  std::iota(order.begin(), order.end(), 0);
  auto ctime = [&](int64_t i) {
    const int w = ent[i].width;
    const double t = w == 128 ? kFusedT[0] : w == 64 ? kFusedT[1] : w == 32 ? kFusedT[2] : kFusedT[3];
    return t * static_cast<double>(ent[i].chunks);
  };
  // (split sequences' chains first: the tail waits for them)
  auto split = [&](int64_t i) { return pl.nseg[ent[i].seq] > 1; };
  std::stable_sort(order.begin(), order.end(), [&](int64_t x, int64_t y) {
    return split(x) != split(y) ? split(x) : ctime(x) > ctime(y);
  });
  f.n_chains = round8(n_ent * H);
  std::vector<int32_t> chains(2 * f.n_chains);
  int64_t c = 0;
  for (int64_t i : order)
    for (int32_t h = 0; h < H; ++h, ++c) {
      chains[2 * c] = static_cast<int32_t>(i);
      chains[2 * c + 1] = h;
    }
  for (; c < f.n_chains; ++c) {
    chains[2 * c] = -1;
    chains[2 * c + 1] = 0;
  }
  // Workgroups: chain << 8 | width code << 4 | tile, the tiles of 8
  // neighbouring chains in rounds so that a chain's tiles share an XCD.
  std::vector<int32_t> wgs;
  auto tiles = [&](int32_t sq) { return ent[sq].kind == 2 ? 1 : dv / ent[sq].width; };
  for (int64_t g = 0; g < f.n_chains / 8; ++g) {
    int rounds = 0;
    for (int x = 0; x < 8; ++x) {
      const int32_t sq = chains[2 * (8 * g + x)];
      if (sq >= 0) rounds = std::max(rounds, tiles(sq));
    }
    for (int r = 0; r < rounds; ++r)
      for (int x = 0; x < 8; ++x) {
        const int64_t ch = 8 * g + x;
        const int32_t sq = chains[2 * ch];
        int code = 15;
        if (sq >= 0 && r < tiles(sq)) {
          const int w = ent[sq].width;
          code = ent[sq].kind == 2 ? 4 : w == 32 ? 0 : w == 64 ? 1 : w == 128 ? 2 : 3;
        }
        wgs.push_back(static_cast<int32_t>((ch << 8) | (code << 4) | (code == 15 ? 0 : r)));
      }
  }
  // Tail items: in the list after every chain (workgroups start in list
  // order, so every chain an item waits for has started when the item
  // starts, and its wait ends).  Last, rather than where the split
  // sequences' chains are predicted to end: the short chains then start
  // before the items, and the items (about 30 us each) fill the launch's
  // end, where a chain of 100 us or more started behind them would not.
  const size_t n_items = titems.size() / kda::kTailInts;
  f.items_fit = n_items < (size_t{1} << 23);
  for (size_t t = 0; t < n_items && f.items_fit; ++t) wgs.push_back(static_cast<int32_t>((t << 8) | (5 << 4)));
  f.n_wg = static_cast<int64_t>(wgs.size());
  // One block: header (word 0: the decay-range flag, zero), then the parts.
  f.w.assign(kHeaderInts, 0);
  auto put = [&](const std::vector<int32_t>& v) {
    const size_t off = f.w.size();
    f.w.insert(f.w.end(), v.begin(), v.end());
    return off;
  };
  f.chains = put(chains);
  f.seqinfo = put(seqinfo);
  f.segx = put(segx);
  f.ck_pos = put(pos);
  f.ck_slot = put(slot);
  f.wgs = put(wgs);
  f.titems = put(titems);
  f.tcnt = put(std::vector<int32_t>(f.n_cnt, 0));
  return f;
}


// The fused launch (split sequences included: their correction is its tail).
int launch_fused_list(const FusedList& fl, const void* q, const void* k, const void* v, const void* a,
                      const void* beta, int32_t H, int32_t dk, int32_t dv, const float* s0, void* o,
                      float* s_final, float* page_pool, int64_t page_elems, void* workspace, int32_t* err_flag,
                      float a_lo, bool gate, float g_min, void* stream) {
  hipStream_t hs = static_cast<hipStream_t>(stream);
  // The work list is staged in pageable host memory: the runtime copies it
  // before hipMemcpyAsync returns (so the call may block the host for that
  // copy), and the vector may then go.
  hipError_t e = hipMemcpyAsync(workspace, fl.w.data(), fl.w.size() * 4, hipMemcpyHostToDevice, hs);
  if (e != hipSuccess) return hip_status(e, "work list copy");
  int32_t* dw = static_cast<int32_t*>(workspace);
  const int64_t hkv = static_cast<int64_t>(H) * dk * dv;
  float* tstate = reinterpret_cast<float*>(static_cast<char*>(workspace) + fl.list_bytes());
  float* xpool = tstate + fl.n_tstate * hkv;
  void* qhat = xpool + fl.n_xpool * hkv;
  const bool cp = fl.n_tstate > 0;
  kda::PrefillArgs p{};
  p.q = q; p.k = k; p.v = v; p.a = a; p.beta = beta;
  p.bf16 = true;
  p.fused = true;
  p.gate = gate;
  p.g_min = g_min;
  p.H = H; p.dk = dk; p.dv = dv; p.chunk = 32;
  p.s0 = s0; p.o = o; p.s_final = s_final;
  p.page_pool = page_pool; p.page_elems = page_elems;
  p.wsflag = dw;
  p.err_flag = err_flag;
  p.a_lo = a_lo;
  p.chains = dw + fl.chains;
  p.seqinfo = dw + fl.seqinfo;
  p.ck_pos = dw + fl.ck_pos;
  p.ck_slot = dw + fl.ck_slot;
  p.wgs = dw + fl.wgs;
  p.n_wg = static_cast<int>(fl.n_wg);
  p.n_chains = static_cast<int>(fl.n_chains);
  p.segx = cp ? dw + fl.segx : nullptr;
  p.titems = dw + fl.titems;
  p.tcnt = dw + fl.tcnt;
  p.qhat = qhat;
  p.xpool = xpool;
  p.tstate = tstate;
  p.stream = hs;
  e = kda::launch_prefill(p);
  if (e != hipSuccess) return hip_status(e, "prefill launch");
  return ok();
}

// Prefill (a_out == nullptr) or segment summaries (a_out != nullptr: q is
// unused, o and s0 are null and s_final receives B; see kda_segment_summary).
int prefill_impl(const void* q, const void* k, const void* v, const void* a, const void* beta,
                 kda_dtype in_dtype, int32_t H, int32_t dk, int32_t dv, int32_t chunk,
                 const int32_t* cu, int32_t n_seqs, const float* s0, void* o, float* s_final,
                 const int32_t* ck_cu, const int32_t* ck_pos, const int32_t* ck_slot,
                 int64_t n_ckpt, float* page_pool, int64_t page_elems, int64_t n_slots,
                 void* workspace, size_t workspace_bytes, int32_t dv_split, float* a_out,
                 int32_t* err_flag, void* stream, bool gate = false, float g_min = 0.f) {
  const bool summary = a_out != nullptr;
  Plan pl;
  int st = make_plan(in_dtype, H, dk, dv, chunk, cu, n_seqs, ck_cu, ck_pos, n_ckpt, dv_split, summary, pl);
  if (st) return st;
  // The decay bound of the chunk form ([Serve demo] §1.3 bounds a to
  // [g_min, 0]): a >= -160/chunk keeps every scaled operand below e^80.
  const float a_lo = -160.f / static_cast<float>(chunk);
  if (gate && (!std::isfinite(g_min) || g_min > 0.f))
    return fail(KDA_EINVAL, "g_min must be finite and <= 0");
  if (gate && g_min < a_lo)
    return fail(KDA_EUNSUPPORTED, "g_min=%g below the decay bound -160/chunk = %g", g_min, a_lo);
  if (n_seqs == 0) return ok();
  const int64_t T = cu[n_seqs];
  const int64_t hkv = static_cast<int64_t>(H) * dk * dv;
  const int64_t hkk = static_cast<int64_t>(H) * dk * dk;

  if (n_ckpt > 0 && (!ck_slot || !page_pool))
    return fail(KDA_EINVAL, "checkpoints need ckpt_slot and page_pool");
  if (n_ckpt > 0) {
    if (page_elems < hkv) return fail(KDA_EINVAL, "page_elems %lld < H*dk*dv %lld",
                                      static_cast<long long>(page_elems), static_cast<long long>(hkv));
    std::unordered_set<int32_t> seen;
    for (int64_t c = 0; c < n_ckpt; ++c) {
      if (ck_slot[c] < 0 || ck_slot[c] >= n_slots)
        return fail(KDA_EINVAL, "checkpoint slot %d outside 0..%lld", ck_slot[c],
                    static_cast<long long>(n_slots) - 1);
      if (!seen.insert(ck_slot[c]).second) return fail(KDA_EINVAL, "checkpoint slot %d repeated", ck_slot[c]);
    }
  }

  // Buffers.
  const size_t es = elem_size(in_dtype);
  if (summary && (!s_final || (n_seqs > 0 && !a_out))) return fail(KDA_EINVAL, "A_out and B_out must not be null");
  if (T > 0 && (!q || !k || !v || !a || !beta || (!summary && !o)))
    return fail(KDA_EINVAL, "null input or output");
  // The kernel reads q, k, a, v as pairs of consecutive elements.
  for (const void* ptr : {q, k, v, a})
    if (reinterpret_cast<uintptr_t>(ptr) % (2 * es))
      return fail(KDA_EINVAL, "q, k, v, a must be aligned to two elements");
  // Output rows are written in 16-byte pieces.
  if (!summary && reinterpret_cast<uintptr_t>(o) % 16) return fail(KDA_EINVAL, "o must be 16-byte aligned");
  if (err_flag && reinterpret_cast<uintptr_t>(err_flag) % 4) return fail(KDA_EINVAL, "err_flag must be aligned");
  const int64_t n_chunks = pl.n_chunks;
  size_t list_bytes = align256(work_ints(n_seqs, H, n_ckpt, n_chunks) * 4);
  size_t need = list_bytes + (pl.fused ? 0 : tile_bytes(n_chunks, H, chunk, dk, es));
  FusedList fl;
  if (pl.fused) {
    // Split sequences only where the workspace holds their buffers (and
    // their tail items can be indexed).
    fl = fused_list(pl, cu, ck_cu, ck_pos, ck_slot, H, dv, s_final != nullptr);
    need = fl.list_bytes() + (fl.n_tstate + fl.n_xpool) * hkv * 4 + align256(fl.n_qrows * H * dk * 2);
    if (pl.cp && (workspace_bytes < need || !fl.items_fit)) {
      st = make_plan(in_dtype, H, dk, dv, chunk, cu, n_seqs, ck_cu, ck_pos, n_ckpt, dv_split, summary, pl, false);
      if (st) return st;
      fl = fused_list(pl, cu, ck_cu, ck_pos, ck_slot, H, dv, s_final != nullptr);
      need = fl.list_bytes();
    }
    list_bytes = fl.list_bytes();
  }
  if (!workspace || workspace_bytes < need)
    return fail(KDA_EWORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(KDA_EINVAL, "workspace must be 256-byte aligned");
  const size_t tok = static_cast<size_t>(T) * H;
  const size_t sbytes = static_cast<size_t>(n_seqs) * hkv * 4;
  const std::vector<Range> ins = {{q, tok * dk * es, "q"}, {k, tok * dk * es, "k"},
                                  {v, tok * dv * es, "v"}, {a, tok * dk * es, "a"},
                                  {beta, tok * es, "beta"}, {s0, s0 ? sbytes : 0, "s0"}};
  const std::vector<Range> outs = {
      {o, summary ? 0 : tok * dv * es, "o"}, {s_final, s_final ? sbytes : 0, summary ? "B_out" : "s_final"},
      {a_out, summary ? static_cast<size_t>(n_seqs) * hkk * 4 : 0, "A_out"},
      {page_pool, n_ckpt > 0 ? static_cast<size_t>(n_slots) * page_elems * 4 : 0, "page_pool"},
      {workspace, need, "workspace"}, {err_flag, err_flag ? 4u : 0u, "err_flag"}};
  st = check_disjoint(outs, ins);
  if (st) return st;
  if (pl.fused) return launch_fused_list(fl, q, k, v, a, beta, H, dk, dv, s0, o, s_final, page_pool, page_elems,
                                         workspace, err_flag, a_lo, gate, g_min, stream);

  // Work list: chains longest sequence first, padded to whole XCD rounds.
  std::vector<int32_t> order(n_seqs);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
    return cu[x + 1] - cu[x] > cu[y + 1] - cu[y];
  });
  const int64_t n_chains = round8(static_cast<int64_t>(n_seqs) * H);
  const int split = pl.split;
  std::vector<int32_t> work(work_ints(n_seqs, H, n_ckpt, n_chunks), 0);
  int32_t* chains = work.data() + kHeaderInts;  // work[0]: the decay-range flag, 0
  int32_t* seqinfo = chains + 2 * n_chains;
  int32_t* wpos = seqinfo + 6 * n_seqs;
  int32_t* wslot = wpos + n_ckpt;
  int32_t* wchunks = wslot + n_ckpt;
  int64_t c = 0;
  for (int32_t s : order)
    for (int32_t h = 0; h < H; ++h, ++c) {
      chains[2 * c] = s;
      chains[2 * c + 1] = h;
    }
  for (; c < n_chains; ++c) {
    chains[2 * c] = -1;
    chains[2 * c + 1] = 0;
  }
  // Chunk table: each sequence's chunks in order, split at its checkpoints.
  int64_t nc = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    const int32_t c0 = ck_cu ? ck_cu[i] : 0, c1 = ck_cu ? ck_cu[i + 1] : 0;
    int32_t* si = seqinfo + 6 * i;
    si[0] = cu[i];
    si[1] = cu[i + 1];
    si[2] = c0;
    si[3] = c1;
    si[4] = static_cast<int32_t>(nc);
    int32_t t = cu[i], c = c0;
    while (t < cu[i + 1]) {
      int32_t e = std::min(t + chunk, cu[i + 1]);
      if (c < c1) e = std::min(e, cu[i] + ck_pos[c]);
      wchunks[2 * nc] = t;
      wchunks[2 * nc + 1] = e - t;
      ++nc;
      if (c < c1 && e == cu[i] + ck_pos[c]) ++c;
      t = e;
    }
    si[5] = static_cast<int32_t>(nc);
  }
  if (nc != n_chunks) return fail(KDA_EINVAL, "internal: chunk count %lld != %lld",
                                  static_cast<long long>(nc), static_cast<long long>(n_chunks));
  for (int64_t i = 0; i < n_ckpt; ++i) {
    wpos[i] = ck_pos[i];
    wslot[i] = ck_slot[i];
  }

  // Mixed launch (slab_mixed_kernel): one entry per workgroup, chain << 8 |
  // width code << 4 | tile, the tiles of 8 neighbouring chains in rounds so
  // that a chain's tiles share an XCD.
  int64_t n_wg = 0;
  int32_t* wgs = wchunks + 2 * n_chunks;
  if (pl.mixed) {
    for (int64_t g = 0; g < n_chains / 8; ++g) {
      int rounds = 0;
      for (int x = 0; x < 8; ++x) {
        const int32_t sq = chains[2 * (8 * g + x)];
        if (sq >= 0) rounds = std::max(rounds, dv / pl.width[sq]);
      }
      for (int r = 0; r < rounds; ++r)
        for (int x = 0; x < 8; ++x) {
          const int64_t ch = 8 * g + x;
          const int32_t sq = chains[2 * ch];
          const int w = sq >= 0 ? pl.width[sq] : 0;
          const int code = w == 32 ? 0 : w == 64 ? 1 : w == 128 ? 2 : 3;
          wgs[n_wg++] = (sq >= 0 && r < dv / w) ? static_cast<int32_t>((ch << 8) | (code << 4) | r)
                                                : static_cast<int32_t>((ch << 8) | (15 << 4));
        }
    }
  }

  hipStream_t hs = static_cast<hipStream_t>(stream);
  // The work list is staged in pageable host memory: the runtime copies it
  // before hipMemcpyAsync returns (so the call may block the host for that
  // copy, a few KB), and the vector may then go.
  hipError_t e = hipMemcpyAsync(workspace, work.data(), work.size() * 4, hipMemcpyHostToDevice, hs);
  if (e != hipSuccess) return hip_status(e, "work list copy");

  int32_t* dwork = static_cast<int32_t*>(workspace);
  kda::PrefillArgs p{};
  p.q = q; p.k = k; p.v = v; p.a = a; p.beta = beta;
  p.bf16 = in_dtype == KDA_BF16;
  p.gate = gate;
  p.slab = pl.slab;
  p.fused = pl.fused;
  p.g_min = g_min;
  p.H = H; p.dk = dk; p.dv = dv; p.chunk = chunk;
  p.s0 = s0; p.o = o; p.s_final = s_final;
  p.page_pool = page_pool; p.page_elems = page_elems;
  p.wsflag = dwork;
  p.err_flag = err_flag;
  p.a_lo = a_lo;
  p.chains = dwork + kHeaderInts;
  p.seqinfo = p.chains + 2 * n_chains;
  p.ck_pos = p.seqinfo + 6 * n_seqs;
  p.ck_slot = p.ck_pos + n_ckpt;
  p.chunks = p.ck_slot + n_ckpt;
  p.n_chunks = static_cast<int>(n_chunks);
  p.tq = static_cast<char*>(workspace) + list_bytes;
  p.n_chains = static_cast<int>(n_chains);
  p.dv_tiles = split;
  p.wgs = p.chunks + 2 * n_chunks;
  p.n_wg = static_cast<int>(n_wg);
  p.stream = hs;
  if (summary) return hip_status(kda::launch_segment_summary(p, a_out, pl.a_split), "segment summary launch");
  return hip_status(kda::launch_prefill(p), "prefill launch");
}

}  // namespace

extern "C" {

int kda_chunk_prefill_workspace_size(int32_t n_seqs, int64_t total_tokens, int32_t H, int32_t dk,
                                     int32_t dv, int32_t chunk, int64_t n_ckpt, kda_dtype in_dtype,
                                     size_t* bytes) {
  if (!bytes) return fail(KDA_EINVAL, "bytes is null");
  if (!valid_dtype(in_dtype)) return fail(KDA_EINVAL, "in_dtype %d", static_cast<int>(in_dtype));
  if (n_seqs < 0 || total_tokens < 0 || H <= 0 || n_ckpt < 0)
    return fail(KDA_EINVAL, "n_seqs=%d total_tokens=%lld H=%d n_ckpt=%lld", n_seqs,
                static_cast<long long>(total_tokens), H, static_cast<long long>(n_ckpt));
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(KDA_EUNSUPPORTED, "dk=%d dv=%d (supported: 16, 32, 64, 128)", dk, dv);
  if (chunk < 16 || chunk > KDA_MAX_CHUNK || chunk % 16)
    return fail(KDA_EUNSUPPORTED, "chunk=%d (a multiple of 16 up to %d)", chunk, KDA_MAX_CHUNK);
  const int64_t mc = max_chunks(n_seqs, total_tokens, chunk, n_ckpt);
  *bytes = align256(work_ints(n_seqs, H, n_ckpt, mc) * 4) +
           (fused_path(in_dtype, dk, chunk) ? 0 : tile_bytes(mc, H, chunk, dk, elem_size(in_dtype)));
  if (fused_path(in_dtype, dk, chunk) && dv == dk) {
    // Room to split long sequences into segments (at most kMaxExtraSegs
    // later segments): their work list, start, end and linear-part states
    // (at most 4 per later segment), checkpoints from zero and from the
    // identity (2 per checkpoint), and qhat (at most one row per token).
    const int64_t n_ent = static_cast<int64_t>(n_seqs) + 2 * kMaxExtraSegs, nch = round8(n_ent * H);
    // (tail items: rows of every token and head, states of every checkpoint
    // and final state and head, each a workgroup entry too)
    const int64_t items =
        2 * kCUs + static_cast<int64_t>(H) * (total_tokens / kTailTokens + 3 * kMaxExtraSegs + n_ckpt);
    const int64_t ints = kHeaderInts + 10 * nch + (6 + kda::kSegxInts) * n_ent + 4 * n_ckpt +
                         (kda::kTailInts + 1) * items + static_cast<int64_t>(H) * kMaxExtraSegs;
    const int64_t hkv = static_cast<int64_t>(H) * dk * dv;
    const size_t cp = align256(static_cast<size_t>(ints) * 4) +
                      static_cast<size_t>(4 * kMaxExtraSegs + 2 * n_ckpt) * hkv * 4 +
                      align256(static_cast<size_t>(total_tokens) * H * dk * 2);
    *bytes = std::max(*bytes, cp);
  }
  return ok();
}

int kda_chunk_prefill_plan(kda_dtype in_dtype, int32_t H, int32_t dk, int32_t dv, int32_t chunk,
                           const int32_t* cu_seqlens_host, int32_t n_seqs, const int32_t* ckpt_cu_host,
                           const int32_t* ckpt_pos_host, int64_t n_ckpt, int32_t dv_split,
                           int32_t* tile_cols_out, char* kernels_out, size_t kernels_bytes) {
  Plan pl;
  const int st = make_plan(in_dtype, H, dk, dv, chunk, cu_seqlens_host, n_seqs, ckpt_cu_host, ckpt_pos_host,
                           n_ckpt, dv_split, false, pl);
  if (st) return st;
  if (tile_cols_out)
    for (int32_t i = 0; i < n_seqs; ++i) tile_cols_out[i] = pl.width[i];
  if (kernels_out && kernels_bytes > 0) {
    const std::string k = plan_kernels(pl, in_dtype, dk, dv, false);
    snprintf(kernels_out, kernels_bytes, "%s", k.c_str());
  }
  return ok();
}

int kda_chunk_prefill_split(const void* q, const void* k, const void* v, const void* a,
                            const void* beta, kda_dtype in_dtype, int32_t H, int32_t dk,
                            int32_t dv, int32_t chunk, const int32_t* cu, int32_t n_seqs,
                            const float* s0, void* o, float* s_final, const int32_t* ck_cu,
                            const int32_t* ck_pos, const int32_t* ck_slot, int64_t n_ckpt,
                            float* page_pool, int64_t page_elems, int64_t n_slots,
                            void* workspace, size_t workspace_bytes, int32_t dv_split,
                            int32_t* err_flag, void* stream) {
  return prefill_impl(q, k, v, a, beta, in_dtype, H, dk, dv, chunk, cu, n_seqs, s0, o, s_final,
                      ck_cu, ck_pos, ck_slot, n_ckpt, page_pool, page_elems, n_slots, workspace,
                      workspace_bytes, dv_split, nullptr, err_flag, stream);
}

int kda_chunk_prefill(const void* q, const void* k, const void* v, const void* a,
                      const void* beta, kda_dtype in_dtype, int32_t H, int32_t dk, int32_t dv,
                      int32_t chunk, const int32_t* cu_seqlens_host, int32_t n_seqs,
                      const float* s0, void* o, float* s_final, const int32_t* ckpt_cu_host,
                      const int32_t* ckpt_pos_host, const int32_t* ckpt_slot_host, int64_t n_ckpt,
                      float* page_pool, int64_t page_elems, int64_t n_slots, void* workspace,
                      size_t workspace_bytes, int32_t* err_flag, void* stream) {
  return kda_chunk_prefill_split(q, k, v, a, beta, in_dtype, H, dk, dv, chunk, cu_seqlens_host,
                                 n_seqs, s0, o, s_final, ckpt_cu_host, ckpt_pos_host,
                                 ckpt_slot_host, n_ckpt, page_pool, page_elems, n_slots, workspace,
                                 workspace_bytes, 0, err_flag, stream);
}

int kda_chunk_prefill_gated(const void* q, const void* k, const void* v, const void* z_a,
                            const void* z_b, float g_min, kda_dtype in_dtype, int32_t H,
                            int32_t dk, int32_t dv, int32_t chunk, const int32_t* cu, int32_t n_seqs,
                            const float* s0, void* o, float* s_final, const int32_t* ck_cu,
                            const int32_t* ck_pos, const int32_t* ck_slot, int64_t n_ckpt,
                            float* page_pool, int64_t page_elems, int64_t n_slots,
                            void* workspace, size_t workspace_bytes, int32_t dv_split,
                            int32_t* err_flag, void* stream) {
  return prefill_impl(q, k, v, z_a, z_b, in_dtype, H, dk, dv, chunk, cu, n_seqs, s0, o, s_final,
                      ck_cu, ck_pos, ck_slot, n_ckpt, page_pool, page_elems, n_slots, workspace,
                      workspace_bytes, dv_split, nullptr, err_flag, stream, true, g_min);
}

int kda_segment_summary_workspace_size(int32_t n_seg, int64_t total_tokens, int32_t H, int32_t dk,
                                       int32_t dv, int32_t chunk, kda_dtype in_dtype,
                                       size_t* bytes) {
  // (the summaries always run the two-kernel path, with its records)
  const int st = kda_chunk_prefill_workspace_size(n_seg, total_tokens, H, dk, dv, chunk, 0, in_dtype, bytes);
  if (st == KDA_OK && fused_path(in_dtype, dk, chunk))
    *bytes += tile_bytes(max_chunks(n_seg, total_tokens, chunk, 0), H, chunk, dk, elem_size(in_dtype));
  return st;
}

int kda_segment_summary(const void* k, const void* v, const void* a, const void* beta,
                        kda_dtype in_dtype, int32_t H, int32_t dk, int32_t dv, int32_t chunk,
                        const int32_t* cu_seg_host, int32_t n_seg, float* A_out, float* B_out,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (n_seg > 0 && !A_out) return fail(KDA_EINVAL, "A_out must not be null");
  if (n_seg == 0) return ok();
  // The summary kernels read no q: the local kernel is handed k in its place.
  return prefill_impl(k, k, v, a, beta, in_dtype, H, dk, dv, chunk, cu_seg_host, n_seg, nullptr,
                      nullptr, B_out, nullptr, nullptr, nullptr, 0, nullptr, 0, 0, workspace,
                      workspace_bytes, 0, A_out, nullptr, stream);
}

}  // extern "C"
