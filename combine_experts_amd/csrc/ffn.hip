// Grouped expert GEMMs over the dispatch buffer (read in place) and the shared
// expert, for decode-sized batches.  "7.13 Serving Mixture-of-Experts",
// section "Expert Parallelism Mechanics", step 3: one grouped GEMM runs all
// local experts' matmuls in a single launch; section "Prefill vs. Decode": at
// decode each expert sees a handful of rows, so the pass is bound by streaming
// the touched experts' weights from HBM.
//
// Design (gfx950):
//  * The weights are the MFMA A operand and go straight from HBM into
//    registers: each step a wave reads 256 bytes of each of its 16 rows.  The
//    activation rows (one 16-token tile per MFMA column block) are the B
//    operand.  Experts with no rows own no work, so their weights are never
//    read.
//  * Work item = (group, 16-row chunk of the group's rows, tile of 16*FW
//    output columns).  Groups are the experts that received rows, in index
//    order, then the shared expert.  Every chunk is an item of its own, so a
//    group with many rows (the shared expert sees all T tokens) is spread
//    over many workgroups that stream the same weights at about the same
//    time, instead of one workgroup walking K once per chunk.  A workgroup
//    has FW x KS waves: FW column tiles, each reduction dimension split KS
//    ways; the KS partial sums are added through LDS in a fixed order
//    (results do not depend on timing or slot order).
//  * Workgroups are persistent: workgroup b of n walks items b, b + n, ...
//    and every wave streams its sequence of (item, K-step) stages through a
//    three-slot register ring, two stages ahead, across item boundaries, so
//    loads stay in flight while an item's epilogue runs.
//    Loads are never skipped (a stage past the end repeats the last address,
//    a token row past a group's end reads the group's first row and its
//    column is never stored), which keeps the wait counts exact.
//  * A CU takes in only so many bytes per microsecond when its loads mix HBM
//    misses with L2 hits, and every column wave needs the same activation
//    tile at a step.  Where the waves of a workgroup walk the same steps,
//    they share that tile through LDS (SHARE, below) instead of each loading
//    it; the launch plan (launch_ffn) picks the shape per pass from the
//    K-steps per item and the rows per touched expert.
//  * The same walk, with one group holding all T tokens and fp32 output, is
//    the router GEMM for 17-2047 tokens (launch_router_gemm).
#include "ffn_body.h"

namespace moe {


template <int DT, int FW, int KS, int TT, bool GATED, int OUT, int NM, bool PARK = true, bool SHARE = false>
__global__ __launch_bounds__(64 * FW * KS) void ffn_kernel(FfnParams p) {
  ffn_body<DT, FW, KS, TT, GATED, OUT, NM, PARK, SHARE>(p, blockIdx.x, gridDim.x);
}

// Residency of the bf16 and f32 walks: one workgroup per CU.  Each wave
// keeps three K-steps of loads in flight, so one workgroup of 2-4 waves
// already draws a CU's share of HBM bandwidth; more resident workgroups only
// add L2 and address-unit contention (measured: 2.5-4% faster on 128-expert
// decode and up to 4% on 256-expert; a cap of two gained nothing).  The cap
// is an unused dynamic LDS reservation sized so a second workgroup cannot
// fit.  The E4M3 walks stay at full occupancy: their dequantising down pass
// measured no better under the cap.
static constexpr int kResidentCap = 1;

template <int DT, int FW, int KS, int TT, bool GATED, int OUT, int NM = 2, bool PARK = true, bool SHARE = false>
static hipError_t launch_one(const FfnParams& p, long long max_items, hipStream_t stream) {
  auto kern = ffn_kernel<DT, FW, KS, TT, GATED, OUT, NM, PARK, SHARE>;
  // constant per kernel and device model: computed once, on the first call
  // (thread-safe initialisation of a const local static)
  static const Residency occ = [&] {
    Residency o{};
    int dev = 0, n = 0, c = 0, lds = 0;
    if (hipGetDevice(&dev) != hipSuccess) return o;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) c = 256;
    if (DT != MOE_FP8_E4M3 && kResidentCap > 0 &&
        hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) == hipSuccess &&
        lds > 0) {
      const size_t r = (size_t)lds / (kResidentCap + 1) + 1;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, 64 * FW * KS, r) == hipSuccess && n >= 1)
        o.reserve = r;
    }
    if (o.reserve == 0 && hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, 64 * FW * KS, 0) != hipSuccess)
      n = 1;
    o.cus = c;
    o.per_cu = n > 0 ? n : 1;
    o.ok = true;
    return o;
  }();
  if (!occ.ok) return hipErrorInvalidDevice;
  const long long cap = (long long)occ.per_cu * occ.cus;
  const int grid = (int)(max_items < cap ? max_items : cap);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * FW * KS), occ.reserve, stream, p);
  return hipGetLastError();
}

// Launch shape of a pass: FW column tiles x KS reduction splits per
// workgroup, 16-row token tiles (one per item).  KS must not exceed the K-steps of any
// item (every wave needs at least one step per item).
struct Plan {
  int fw, ks;
};

static Plan plan_of(const FfnParams& p, int step, bool gated, int wdtype) {
  int steps = p.K_r / step;
  if (p.n_shared && p.K_s / step < steps) steps = p.K_s / step;
  // Long reductions are split over 4 waves (keeps enough waves busy when few
  // experts have rows); shorter ones keep more steps per wave instead.
  Plan pl{1, 4};
  if (steps < 32) pl = steps >= 8 ? Plan{2, 2} : Plan{gated ? 4 : 2, 1};
  if (steps < pl.ks) pl = Plan{gated ? 4 : 2, 1};
  if (gated && wdtype == MOE_FP8_E4M3) pl = Plan{8, 1};
  return pl;
}

template <int DT, bool GATED, int OUT, int TT = 1, bool PARK = true, bool SHARE = false>
static hipError_t launch_plan(const FfnParams& p, const Plan& pl, long long items, hipStream_t stream) {
#define MOE_FFN_CASE(FW, KS)           \
  if (pl.fw == FW && pl.ks == KS)      \
    return launch_one<DT, FW, KS, TT, GATED, OUT, 2, PARK, SHARE>(p, items, stream);
  MOE_FFN_CASE(1, 4)
  MOE_FFN_CASE(1, 2)
  MOE_FFN_CASE(1, 1)
  MOE_FFN_CASE(8, 1)
  MOE_FFN_CASE(4, 1)
  MOE_FFN_CASE(2, 2)
  MOE_FFN_CASE(2, 1)
#undef MOE_FFN_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_ffn(const FfnParams& p, int wdtype, bool gated, long long routed_rows, int max_groups,
                      hipStream_t stream) {
  const int step = wdtype == MOE_F32 ? 64 : wdtype == MOE_BF16 ? 128 : 256;
  if (p.K_r / step < 1 || (p.n_shared && p.K_s / step < 1)) return hipErrorInvalidValue;
  Plan pl = plan_of(p, step, gated, wdtype);
  // E4M3 batches with at least one row per expert on average (T k >= E) use
  // wide chunks (64 rows where the launch shape allows, below; else 32): each
  // weight tile is then streamed once per 64 rows instead of once per 16.  The
  // wider activation tiles leave no registers for parked accumulators, so
  // those walks finish each item in line.  Measured layer us against 16-row
  // chunks, 8 of 256 experts, two runs each on one box: 16 tokens 690 / 685
  // (below the rule), 32 964 / 1007, 48 1092 / 1131, 64 1184 / 1168, 80 1213 /
  // 1250, 96 1314 / 1363, 128 1426 / 1449, 256 1589 / 1780.
  const bool wide = wdtype == MOE_FP8_E4M3 && p.E > 0 && routed_rows >= p.E;
  // Once experts hold a few rows each, the E4M3 down pass does better with
  // more column waves sharing each activation tile and no K-split.  Measured
  // at 256 experts x 8 slots, down pass with (2, 2) / (4, 1) / (8, 1): 512
  // tokens 782 / 710 / 686 us; 128 tokens 506 / 489 / 494 us; 32 tokens (one
  // row per expert) 322 / 326 / 335 us.
  if (!gated && wdtype == MOE_FP8_E4M3 && routed_rows >= 2LL * max_groups) {
    for (const Plan w : {wide ? Plan{8, 1} : Plan{4, 1}, Plan{4, 1}})
      if (p.tiles_r % (2 * w.fw) == 0 && p.tiles_s % (2 * w.fw) == 0) {
        pl = w;
        break;
      }
  }
  // A bf16 gated pass of 16-31 steps with under two rows per touched expert
  // and at least 32 of them: one column wave per item and a 4-way K-split.
  // Measured at 128 experts x 8 slots, d_model = 2048, (2, 2) against (1, 4),
  // two runs each: 8 tokens 62.1, 62.3 / 58.7, 59.1 us.  It loses at 1 token
  // (8 experts: 19.3, 19.5 / 20.8, 20.1 us) and from 32 tokens on (126.5,
  // 126.3 / 131.4, 131.5 us; 128 tokens 141.9, 142.2 / 153.8, 153.9 us).
  // Not with a shared expert, whose items moe_layer may run in the router's
  // launch with the shape of plan_of.
  if (gated && wdtype == MOE_BF16 && !p.n_shared && max_groups >= 32 && routed_rows < 2LL * max_groups &&
      p.K_r / step >= 16 && p.K_r / step < 32)
    pl = Plan{1, 4};
  // A bf16 plain pass with short items (under 16 steps) and eight or more
  // rows per touched expert: four column waves sharing each activation tile.
  // Measured at 128 experts x 8 slots, d_ff = 768 (6 steps), down pass with
  // (2, 1) private / (4, 1) shared tiles, two runs each: 128 tokens
  // 80.7, 81.3 / 78.7, 78.5 us; 256 tokens 108.5, 109.3 / 99.5, 100.0 us.
  // With fewer rows per expert the tiles are mostly padding and sharing them
  // does not pay (32 tokens: 67.7 against 71.6 us).
  const bool dense_plain = !gated && wdtype == MOE_BF16 && routed_rows >= 8LL * max_groups;
  if (dense_plain) {
    int st = p.K_r / step;
    if (p.n_shared && p.K_s / step < st) st = p.K_s / step;
    if (st < 16 && p.tiles_r % 8 == 0 && p.tiles_s % 8 == 0) pl = Plan{4, 1};
  }
  // a work item covers FW waves' columns; a plain-pass wave covers two tiles
  const int per_item = pl.fw * (gated ? 1 : 2);
  FfnParams q = p;
  q.tiles_r = p.tiles_r / per_item;
  q.tiles_s = p.tiles_s / per_item;
  if (q.tiles_r * per_item != p.tiles_r || q.tiles_s * per_item != p.tiles_s) return hipErrorInvalidValue;
  // Those batches take 64-row chunks where the launch shape allows (the
  // gated pass, and the down pass without a K-split): a group of 33-64 rows
  // then streams its weight tiles once instead of twice.  Measured at 512
  // tokens x 8 of 256 experts against 32-row chunks: gate/up 1280 -> 1195 us,
  // down 666 -> 629 us, layer 2072 -> 1936 us.
  const bool wide64 = wide && (gated || (pl.ks == 1 && (pl.fw == 8 || pl.fw == 4)));
  const int CH = wide64 ? 64 : wide ? 32 : 16;
  // CH-row chunks over all groups: full chunks plus at most one partial
  // chunk per group (bounds the items, which sizes the grid)
  const long long chunks_r = routed_rows / CH + max_groups;
  const long long chunks_s = q.n_shared ? (q.T + CH - 1) / CH : 0;
  const long long items = chunks_r * q.tiles_r + chunks_s * q.tiles_s;
  if (items <= 0) return hipSuccess;
  if (wdtype == MOE_F32) {
    if (gated) return launch_plan<MOE_F32, true, MOE_F32>(q, pl, items, stream);
    return launch_plan<MOE_F32, false, MOE_F32>(q, pl, items, stream);
  }
  // every wave of a workgroup walks the same number of steps per item
  const bool even = (q.K_r / step) % pl.ks == 0 && (!q.n_shared || (q.K_s / step) % pl.ks == 0);
  if (wdtype == MOE_BF16) {
    // bf16 tiles are shared between column waves of items with 16 or more
    // steps: measured at 128 tokens, 128 experts: gate/up (16 steps) 143.0 ->
    // 141.5 us, but the 6-step down pass with (2, 1) 80.4 -> 84.2 us; 256
    // experts: down (16 steps) 941 -> 916 us.  Short dense plain passes share
    // under the (4, 1) shape chosen above.
    int steps = q.K_r / step;
    if (q.n_shared && q.K_s / step < steps) steps = q.K_s / step;
    const bool dense4 = dense_plain && pl.fw == 4 && pl.ks == 1;
    if ((pl.fw >= 2 && steps >= 16 && even) || dense4) {
      if (gated) return launch_plan<MOE_BF16, true, MOE_BF16, 1, true, true>(q, pl, items, stream);
      return launch_plan<MOE_BF16, false, MOE_F32, 1, true, true>(q, pl, items, stream);
    }
    if (gated) return launch_plan<MOE_BF16, true, MOE_BF16>(q, pl, items, stream);
    return launch_plan<MOE_BF16, false, MOE_F32>(q, pl, items, stream);
  }
  if (wide64) {
    if (gated) return launch_one<MOE_FP8_E4M3, 8, 1, 4, true, MOE_FP8_E4M3, 2, false, true>(q, items, stream);
    if (pl.fw == 8) return launch_one<MOE_FP8_E4M3, 8, 1, 4, false, MOE_F32, 2, false, true>(q, items, stream);
    return launch_one<MOE_FP8_E4M3, 4, 1, 4, false, MOE_F32, 2, false, true>(q, items, stream);
  }
  if (wide) {
    // The waves of a workgroup share each step's 32-row activation tile
    // through LDS (measured upper bound, with the activation loads removed
    // altogether at 512 tokens: gate/up 1803 -> 1229 us, down 923 -> 717 us).
    // Sharing needs every wave to walk the same number of steps per item, so
    // the K-split must divide every item's steps.
    if (gated) return launch_one<MOE_FP8_E4M3, 8, 1, 2, true, MOE_FP8_E4M3, 2, false, true>(q, items, stream);
    if (even) return launch_plan<MOE_FP8_E4M3, false, MOE_F32, 2, false, true>(q, pl, items, stream);
    return launch_plan<MOE_FP8_E4M3, false, MOE_F32, 2, false>(q, pl, items, stream);
  }
  // 16-row chunks share their tiles too (measured upper bound at 128 tokens:
  // gate/up 1005 -> 932 us, down 534 -> 488 us)
  if (gated) return launch_one<MOE_FP8_E4M3, 8, 1, 1, true, MOE_FP8_E4M3, 2, true, true>(q, items, stream);
  if (even) return launch_plan<MOE_FP8_E4M3, false, MOE_F32, 1, true, true>(q, pl, items, stream);
  return launch_plan<MOE_FP8_E4M3, false, MOE_F32>(q, pl, items, stream);
}

// The router GEMM at decode: its weight is small (E x d), so an item is one
// 16-column tile (NM = 1) and the reduction is split eight ways inside the
// workgroup, which spreads it over E / 16 workgroups of eight waves.
template <int DT>
static hipError_t launch_router_dt(const FfnParams& q, long long items, int steps, hipStream_t stream) {
  if (steps >= 8) return launch_one<DT, 1, 8, 1, false, MOE_F32, 1>(q, items, stream);
  if (steps >= 4) return launch_one<DT, 1, 4, 1, false, MOE_F32, 1>(q, items, stream);
  return launch_one<DT, 1, 1, 1, false, MOE_F32, 1>(q, items, stream);
}

hipError_t launch_router_gemm(const FfnParams& p, int dtype, hipStream_t stream) {
  const int step = dtype == MOE_F32 ? 64 : 128;
  if (p.E != 0 || !p.masked || p.n_shared != 1 || p.Nout_s % 16 || p.K_s % step) return hipErrorInvalidValue;
  FfnParams q = p;
  q.tiles_r = 0;
  q.tiles_s = p.Nout_s / 16;
  const long long items = (long long)(p.T + 15) / 16 * q.tiles_s;
  const int steps = p.K_s / step;
  if (dtype == MOE_F32) return launch_router_dt<MOE_F32>(q, items, steps, stream);
  if (dtype == MOE_BF16) return launch_router_dt<MOE_BF16>(q, items, steps, stream);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// The router next to the shared expert's gate/up pass, in one launch
// ("Hot-Expert Skew" section, shared experts; the shared expert needs no
// routing).  The first nroute workgroups route four tokens each (one, and
// write it, in the masked layout); the others run the persistent gate/up
// walk over the shared expert's items only (sp has no routed groups),
// streaming its weights while HBM would otherwise idle behind the router.  bf16 only: on the E4M3 path the shared expert reads the
// tokens the dispatch quantises.
// ---------------------------------------------------------------------------

template <int KPL, int FW, int KS>
__global__ __launch_bounds__(64 * FW * KS) void route_shared_kernel(RouteParams rp, FfnParams sp, int nroute) {
  extern __shared__ float smem[];
  static_assert(FW * KS == 4, "the routing workgroups hold four waves");
  if ((int)blockIdx.x < nroute) {
    if (rp.fuse) route_dispatch_block<KPL>(rp, blockIdx.x, smem);  // one token, masked-layout write
    else route_body<KPL, 4>(rp, blockIdx.x, smem);                 // four tokens
  } else
    ffn_body<MOE_BF16, FW, KS, 1, true, MOE_BF16, 2>(sp, blockIdx.x - nroute, gridDim.x - nroute);
}

template <int KPL, int FW, int KS>
static hipError_t launch_rs(const RouteParams& rp, const FfnParams& q, long long items, hipStream_t stream) {
  auto kern = route_shared_kernel<KPL, FW, KS>;
  constexpr int NT = 64 * FW * KS;
  const size_t lds = (size_t)(FW * KS) * route_lds_floats(rp.E) * sizeof(float);
  // workgroups per CU for the largest routing LDS (E = 1024), constant per
  // kernel and device model: computed once (thread-safe static initialisation)
  static const Residency occ = [&] {
    Residency o{};
    int dev = 0, n = 0, c = 0;
    if (hipGetDevice(&dev) != hipSuccess) return o;
    const size_t lds_max = (size_t)(FW * KS) * route_lds_floats(1024) * sizeof(float);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, NT, lds_max) != hipSuccess || n < 1) n = 1;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) c = 256;
    o.per_cu = n;
    o.cus = c;
    o.ok = true;
    return o;
  }();
  if (!occ.ok) return hipErrorInvalidDevice;
  const long long cap = (long long)occ.per_cu * occ.cus;
  const int nroute = rp.fuse ? rp.T : (rp.T + FW * KS - 1) / (FW * KS);
  const int nshared = (int)(items < cap ? items : cap);
  hipLaunchKernelGGL(kern, dim3(nroute + nshared), dim3(NT), lds, stream, rp, q, nroute);
  return hipGetLastError();
}

bool route_shared_supported(const FfnParams& sp, int wdtype) {
  if (wdtype != MOE_BF16 || !sp.n_shared) return false;
  const Plan pl = plan_of(sp, 128, true, wdtype);
  return (pl.fw == 1 && pl.ks == 4) || (pl.fw == 2 && pl.ks == 2);
}

hipError_t launch_route_shared(const RouteParams& rp, const FfnParams& sp, int wdtype, hipStream_t stream) {
  if (!route_shared_supported(sp, wdtype)) return hipErrorInvalidValue;
  const Plan pl = plan_of(sp, 128, true, wdtype);
  FfnParams q = sp;
  q.E = 0;  // no routed groups: the walk covers the shared expert only
  q.tiles_r = sp.tiles_r / pl.fw;
  q.tiles_s = sp.tiles_s / pl.fw;
  if (q.tiles_s * pl.fw != sp.tiles_s) return hipErrorInvalidValue;
  const long long items = (long long)(q.T + 15) / 16 * q.tiles_s;
  const int kpl = (rp.E + 63) / 64;
#define MOE_RS_CASE(K)                                                          \
  if (kpl <= K) {                                                               \
    if (pl.fw == 1) return launch_rs<K, 1, 4>(rp, q, items, stream);            \
    return launch_rs<K, 2, 2>(rp, q, items, stream);                            \
  }
  MOE_RS_CASE(1)
  MOE_RS_CASE(2)
  MOE_RS_CASE(4)
  MOE_RS_CASE(8)
  MOE_RS_CASE(16)
#undef MOE_RS_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe
