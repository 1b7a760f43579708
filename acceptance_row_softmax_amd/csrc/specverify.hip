// libspecverify: speculative-decoding verification kernels for gfx950 and the C ABI
// declared in include/specverify.h.
//
// Linear drafts: one launch per call. Its workgroups hold two independent waves;
// in dispatch order:
//  * greedy: one streaming wave per (target row, 8 KiB chunk), rows in position
//    order, each writing its chunk's max and lowest argmax as a tagged record; then
//    one finishing wave per sequence, which reads its rows' records, takes L as the
//    first draft that is not its row's argmax and writes the outputs.
//  * stochastic: for each position i < k and each sequence, the streaming waves of
//    rows t_i and d_i (each writes its chunk's max, softmax weight sum and the draft
//    token's logit as a tagged record and ends), then the pair's finishing wave,
//    which polls those records: it combines both rows, runs
//    the acceptance test u_i < p_t,i(x_i) / p_d,i(x_i) and records the outcome in
//    the sequence's state word; the update that settles the first rejected position
//    L hands rows t_L, d_L to the residual waves. Then, per sequence, the streaming
//    waves of target row k, that row's finishing wave (the bonus draw) and two
//    residual waves per chunk: each sums max(0, p_t,L - p_d,L) over its half
//    chunk; the last of a sequence picks the part holding u*S, and the correction
//    token is drawn by an inverse-CDF scan inside it (by the wave that holds that
//    part in hold mode, else after a reload). A launch with more residual waves
//    than the GPU keeps waiting at once is queued: its residual waves serve
//    decision slots taken in the order the decisions are made, rejections first,
//    the first slots' waves ahead of target row k's stream and the others last;
//  * one wave writes all outputs of a sequence: the wave that drew its correction
//    token, once the sequence's other events (an atomic counter per sequence) have
//    all counted; with every draft accepted, the last event to count. A wave that
//    drew the final token with L settled issues the emission's reads early.
// No wave ever waits for work dispatched after it: finishing waves wait for the
// streaming waves before them, residual waves for decisions and events of
// finishing waves before them, and a last event only for a token whose wave has
// already counted itself. Every wait is bounded in time.
//
// Trees: a streaming launch of the same kind reduces every node's row (greedy:
// its argmax is the node's token; stochastic: for a small batch the token is
// drawn there too, at every node). Trees of at most 256 nodes whose tokens are
// then known are walked in that launch, by the wave that combines the tree's last
// node; otherwise a second launch runs one workgroup per tree that searches the
// accepted path in LDS, and for a large stochastic batch walks level by level and
// draws the tokens of the accepted nodes only. Row statistics: the streaming
// launch alone.
//
// Sources: "Accelerating Sonar through speculation" (sections "Spekulatives
// Decoding", "Ziel-Entwurf", "MTP", "EAGLE"); "Speculative-Decoding, LLM推理的加速 /
// Medusa 方法阅读" (section 三). The acceptance rule is that of the Leviathan et al.
// method the Sonar page cites: accept x_i iff u_i < p_t,i(x_i) / p_d,i(x_i).
#include "../../include/specverify.h"
#include "sv_device.hpp"
#include "sv_host.hpp"
#include "sv_rows.hpp"

#include <hip/hip_runtime.h>
#include <algorithm>
#include <atomic>
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <mutex>

using namespace sv;

// Workspace of spec_verify_linear_static, one copy per GPU. In host code the name
// stands for the host-side shadow, not a device address: only the address from
// hipGetSymbolAddress (static_scratch()) is ever passed to a kernel or a fill.
static __device__ __align__(256) unsigned char scratch[SV_MAX_STATIC_WORKSPACE];

namespace {

constexpr double LN2 = 0.69314718055994530941723212145818;


// What the residual waves of a sequence need. kind 0: no draft rejected (the bonus
// token is final); 1: draw from the residual of rows t_L, d_L; 2: a draft was
// rejected but its rows are unusable (data error, no draw). b is the sequence (the
// residual waves of a queued launch learn it from here).
struct Decision {
  int16_t L;
  int16_t kind;
  int32_t b;
  float Mt, Md;
  double Zt, Zd;
};
constexpr int DEC_WORDS = RecWords<Decision>::N;   // 8

// Statistics of the (target, draft) row pair of one position, kept for the wave
// that settles the first rejected position when that is another position.
struct PairStat {
  double Zt, Zd;
  float Mt, Md;
  int okt, okd;
};
constexpr int PST_WORDS = RecWords<PairStat>::N;   // 8

struct ResPart {
  double s;
};
constexpr int RES_WORDS = RecWords<ResPart>::N;    // 2

struct Token {
  int y;        // -1 no token (data error), -2 a wait timed out
};

struct Probs {  // p_t,i(x_i) and p_d,i(x_i) of one position (stochastic)
  float pt, pd;
};
constexpr int PROB_WORDS = RecWords<Probs>::N;    // 2

// Sequence state word: bit i (i < k) position i decided, bit 32+i position i
// rejected, BONUS_BIT the bonus row has been drawn.
constexpr uint64_t BONUS_BIT = 1ull << 31;

// First rejected position if the state fixes it, k if every draft is accepted and
// the bonus row is drawn, else -1.
__device__ __forceinline__ int settled_L(uint64_t s, int k) {
  const uint64_t mk = (1ull << k) - 1;
  const uint64_t dec = s & mk, rej = (s >> 32) & mk;
  const int fr = rej ? __builtin_ctzll(rej) : k;
  const uint64_t und = ~dec & mk;
  const int fu = und ? __builtin_ctzll(und) : k;
  if (fr < k) return fu > fr ? fr : -1;
  return (fu == k && (s & BONUS_BIT)) ? k : -1;
}


__device__ __forceinline__ ResidW make_residw(const Decision& d, float c0) {
  ResidW rw;
  rw.c0 = c0;
  rw.mc0t = d.Mt * c0;
  rw.mc0d = d.Md * c0;
  // 1 / sum_v exp2(x_v*c0 - fl32(M*c0)), from Z = sum_v exp2(x_v*c0 - M*c0)
  rw.izt = (float)(1.0 / (d.Zt * exp2((double)d.Mt * (double)c0 - (double)rw.mc0t)));
  rw.izd = (float)(1.0 / (d.Zd * exp2((double)d.Md * (double)c0 - (double)rw.mc0d)));
  return rw;
}

// Residual waves take half a chunk each (RH parts of HU units per lane): two rows'
// halves are 32 registers per lane, where whole chunks would be 64, which would
// set the occupancy of the whole launch.
constexpr int RH = 2;
constexpr int64_t EARLY_SLOTS = 32;   // queued launches: see linear_setup
constexpr int HU = CU / RH;

// Residual sum over a loaded run of units of rows t_L, d_L (same value in every
// lane); us receives this lane's unit sums, as the in-run search forms them.
template <int DT, int NU>
__device__ __forceinline__ double residual_raw_sum(const RawN<NU>& rt, const RawN<NU>& rd, const ResidW& rw,
                                                   float (&us)[NU]) {
  chunk_unit_sums<DT, true>(rt, rd, rw, us);
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < NU; ++j) s += (double)us[j];
  return wave_sum(s);
}

// The last residual wave's verdict on one part, for the wave holding it (hold
// mode): kind 0 not picked, 1 picked (draw from the residual), 2 picked with no
// residual mass (draw from p_t,L); th the threshold inside the part; fo the
// sequence's event count as the last residual wave read it with the part sums
// (the drawing wave polls it again only if some other event had not counted).
struct Verdict {
  int kind;
  uint32_t fo;
  double th;
};
constexpr int VERD_WORDS = RecWords<Verdict>::N;   // 4

// ------------------------------------------------------------------ linear drafts
// Streaming waves: one per 8 KiB chunk of a row. A streaming wave reduces its
// chunk to a partial, writes it as the chunk's record with a single store
// instruction (lane j stores word j) and ends without waiting for it. Every word of
// a record is a 32-bit value with the call's 32-bit tag (see put_rec):
//   stochastic: word 0 the chunk's max (f32 bits), words 1 and 2 the low and high
//               halves of its f64 weight sum relative to fl32(max*c0), word 3 the
//               row's draft-token logit if the chunk holds that token, else
//               NOT_HELD (a NaN pattern no decoded logit has)
//   greedy:     word 0 the chunk's max, word 1 its lowest argmax
// A combine group is finished by a wave of its own, dispatched after the group's
// chunks: it polls the group's records (each lane its chunks' words) until every
// word carries the call's tag, and clears them behind the read. Counting each
// chunk into a group counter and polling that instead measured slower: a
// streaming wave with a store or atomic still in flight holds its slot, and the
// counter adds a round trip before the records are read. Groups:
// greedy, every chunk of a sequence; stochastic, the target and draft rows of one
// position (the pair finish runs that position's acceptance test), and the target
// row after the last draft (the bonus draw).
struct LinearParams {
  const char* target;
  const char* draft;
  const int32_t* tokens;
  const float* uniforms;
  int32_t* accept_len;
  int32_t* out_tokens;
  float* p_target;
  float* p_draft;
  int32_t* err_flags;
  uint64_t* seg;        // [RQ][C][RW] chunk records
  uint64_t* pst;        // [B][k]   PairStat records (stochastic)
  uint64_t* rks;        // [B]      RowStat records of target rows k (stochastic)
  uint64_t* dec;        // [B][CG]  Decision records, one copy per residual wave (queued: [slot][CG])
  uint64_t* res;        // [B][CG]  ResPart records
  uint64_t* verd;       // [B][CG]  Verdict records (hold mode)
  uint64_t* tok;        // [B]      Token records
  uint64_t* prob;       // [B][k]   Probs records (stochastic)
  uint64_t* state;      // [B]      sequence state words (stochastic)
  uint32_t* fin;        // [B]      events per sequence (stochastic)
  uint32_t* res_cnt;    // [B]      residual waves done per sequence
  uint32_t* errw;       // [B]      error bits per sequence
  uint64_t* slots;      // [1]      queued: decisions placed so far, rejections (low half) and acceptances (high half)
  int64_t B, k, V;
  int C;                // chunks per row
  int CG;               // residual waves per sequence: RH per chunk
  int RW;               // words per chunk record
  int EV;               // events per sequence (stochastic): k pair combines, target row k, the final token
  bool hold;            // residual waves keep their part until the draw is placed (see linear_residual_wave)
  bool queue;           // residual waves serve decision slots, not sequences (see publish_decision)
  float c0;
  uint32_t tag;
  int64_t n_waves;      // waves of the launch (see linear_role)
  uint32_t tk0;         // stochastic: first wave after the position blocks (see linear_role)
  uint32_t early;       // residual waves before the sequence blocks: hold mode every sequence's, queued the first slots'
  // optional commit by the emitting wave (spec_verify_linear_commit)
  int32_t* seq_len;     // [B] in/out
  int32_t* history;     // [B][capacity]
  int64_t capacity;
  int32_t* shifted;     // [B][k+1]
  int32_t* next_token;  // [B]
  bool commit;
};

// Row order. Stochastic: q = i*2B + 2b + which for i < k (which 0 target, 1
// draft), q = 2kB + b for target row k. Greedy: q = i*B + b.
template <bool STOCH>
__device__ __forceinline__ int64_t row_q(const LinearParams& P, int64_t b, int64_t i, int which) {
  if (!STOCH) return i * P.B + b;
  if (i < P.k) return i * 2 * P.B + 2 * b + which;
  return 2 * P.k * P.B + b;
}

template <bool STOCH>
__device__ __forceinline__ void row_of_q(const LinearParams& P, uint32_t q, int64_t& b, int64_t& i, int& which) {
  if constexpr (STOCH) {
    const uint32_t twoB = (uint32_t)(2 * P.B);
    const uint32_t pairs = (uint32_t)P.k * twoB;
    if (q < pairs) {
      i = q / twoB;
      const uint32_t rem = q - (uint32_t)i * twoB;
      b = rem >> 1;
      which = (int)(rem & 1u);
    } else {
      i = P.k;
      b = q - pairs;
      which = 0;
    }
  } else {
    const uint32_t B32 = (uint32_t)P.B;
    i = q / B32;
    b = q - (uint32_t)i * B32;
    which = 0;
  }
}

template <int DT, bool STOCH>
__device__ __forceinline__ const char* row_ptr(const LinearParams& P, int64_t b, int64_t i, int which) {
  constexpr int E = DTraits<DT>::E;
  if (which) return P.draft + ((b * P.k + i) * P.V) * E;
  return P.target + ((b * (P.k + 1) + i) * P.V) * E;
}

__device__ __forceinline__ uint64_t seg_load(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void seg_store(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t tagged(uint32_t v, uint32_t tag) { return ((uint64_t)tag << 32) | v; }

constexpr uint32_t NOT_HELD = 0x7fffffffu;

// The chunk partials of NR consecutive rows q0, q0+1 (stochastic records; lane l
// holding chunks l + 64 t of each row, and the draft token's logit if some chunk of
// the row holds it), each word polled until it carries the call's tag (clear_rows
// zeroes them afterwards).
// One round of 64 chunks at a time (for both rows), so that only one round's words
// are held; every round's wait counts against the same time limit. false on timeout.
// If sp is given, lane 0 reads that sequence state word with every poll, so that
// *sv is the state as it was when the last records arrived.
template <int NR>
__device__ __forceinline__ bool read_rows(const LinearParams& P, int64_t q0, RowParts (&rp)[NR],
                                          const uint64_t* sp = nullptr, uint64_t* sv = nullptr) {
  const int lane = lane_id();
  bool ok = true;
  WaitClock clk;
  int xin[NR];
  uint32_t xv[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    xin[r] = 0;
    xv[r] = 0;
  }
#pragma unroll
  for (int t = 0; t < MAX_ROUNDS; ++t) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      rp[r].m[t] = -INFINITY;
      rp[r].idx[t] = INT_SENTINEL;
      rp[r].s[t] = 0.0;
    }
    if (t * WAVE >= P.C) continue;
    const int c = t * WAVE + lane;
    const bool in = c < P.C;
    uint64_t w[NR][4];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) w[r][e] = 0;
    bool got = false;
    for (bool go = ok; go && !got;) {   // after a timeout, later rounds are not waited for
      if (sp && lane == 0) *sv = state_load(sp);
      bool mine = true;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if (in) {
          const uint64_t* q = P.seg + ((q0 + r) * P.C + c) * P.RW;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            w[r][e] = seg_load(q + e);
            mine = mine && (uint32_t)(w[r][e] >> 32) == P.tag;
          }
        }
      }
      got = __ballot(!mine) == 0ull;
      if (!got) {
        go = clk.more();
        __builtin_amdgcn_s_sleep(2);
      }
    }
    ok = ok && got;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if (in) {
        rp[r].m[t] = __uint_as_float((uint32_t)w[r][0]);
        rp[r].s[t] = __longlong_as_double((long long)(((uint64_t)(uint32_t)w[r][2] << 32) | (uint32_t)w[r][1]));
        if ((uint32_t)w[r][3] != NOT_HELD) {
          xin[r] = 1;
          xv[r] = (uint32_t)w[r][3];
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const unsigned long long xm = __ballot(xin[r] != 0);
    rp[r].xin = xm != 0ull;
    rp[r].xv = __uint_as_float((uint32_t)__shfl((int)xv[r], xm ? first_lane(xm) : 0));
    rp[r].got = ok;
  }
  return ok;
}

// Zeroes the chunk records of NR consecutive rows from q0 for the next call (lane l:
// chunks l + 64 t), once the wave has nothing left to wait for: a wait for a load
// or a returning atomic also waits for every store issued before it, and these
// device-scope stores take about a microsecond to complete.
template <int NR>
__device__ __forceinline__ void clear_rows(const LinearParams& P, int64_t q0) {
  const int lane = lane_id();
#pragma unroll
  for (int r = 0; r < NR; ++r)
    for (int c = lane; c < P.C; c += WAVE) {
      uint64_t* q = P.seg + ((q0 + r) * P.C + c) * P.RW;
#pragma unroll
      for (int e = 0; e < 4; ++e) store_zero(q + e);
    }
}

constexpr int TOKEN_UNKNOWN = INT_SENTINEL;

// What the emission of sequence b reads (per lane), and the reading: issued as
// soon as the emitting wave knows it is last, so that it can overlap a draw.
struct EmitIn {
  uint64_t s;
  uint32_t ew;
  Token t;
  bool tg, pg;
  int x;
  Probs pr;
};

template <int DT, bool STOCH>
__device__ __forceinline__ EmitIn emit_load(const LinearParams& P, int64_t b, bool token_known) {
  const int lane = lane_id();
  const int64_t k = P.k;
  EmitIn in;
  in.s = 0;
  in.ew = 0;
  in.t.y = -2;
  in.tg = true;
  in.pg = true;
  if (lane == 0) in.s = state_load(P.state + b * SSTRIDE);
  if (lane == 1) in.ew = __hip_atomic_load(P.errw + b * CSTRIDE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (lane == 2 && !token_known) in.tg = get_rec(P.tok + b, in.t, P.tag);
  const bool has = lane < k;
  in.x = has ? P.tokens[b * k + lane] : 0;
  in.pr.pt = in.pr.pd = NAN;
  if (STOCH && has) in.pg = get_rec(P.prob + (b * k + lane) * PROB_WORDS, in.pr, P.tag);
  return in;
}

// Leaves sequence b's words and records zero for the next call (stochastic). Issued
// after the outputs: a wait for a load also waits for every store the wave issued
// before it, and these device-scope stores take about a microsecond to complete,
// so issued first they delayed every emission by that much (a read of the error
// word, whose place among the wave's memory operations the compiler cannot count,
// made it wait for all of them).
__device__ __forceinline__ void emit_clear(const LinearParams& P, int64_t b, bool token_rec) {
  const int lane = lane_id();
  const int64_t k = P.k;
  if (lane < k) {
    clear_rec<Probs>(P.prob + (b * k + lane) * PROB_WORDS);
    clear_rec<PairStat>(P.pst + (b * k + lane) * PST_WORDS);
  }
  if (lane == 0) counter_reset(P.state + b * SSTRIDE);
  if (lane == 1) counter_reset(P.errw + b * CSTRIDE);
  if (lane == 2 && token_rec) clear_rec<Token>(P.tok + b);
  if (lane == 3) clear_rec<RowStat>(P.rks + b * ROW_WORDS);
  if (lane == 4) counter_reset(P.fin + b * CSTRIDE);
}

// Writes every output of sequence b (by its one emitting wave): the first rejected
// position from the state word, the final token (known_y, or the token record),
// the error bits, and the accepted drafts. One writer per output.
template <int DT, bool STOCH>
__device__ __forceinline__ void emit_store(const LinearParams& P, int64_t b, const EmitIn& in, int known_y) {
  const int lane = lane_id();
  const int64_t k = P.k, V = P.V;
  const bool has = lane < k;
  const uint64_t s = __shfl(in.s, 0);
  int err = (int)__shfl(in.ew, 1);
  const int y = known_y != TOKEN_UNKNOWN ? known_y : __shfl(in.tg ? in.t.y : -2, 2);
  const uint64_t rej = (s >> 32) & ((1ull << k) - 1);
  const int L = rej ? __builtin_ctzll(rej) : (int)k;
  if (__ballot(has && (in.x < 0 || in.x >= V))) err |= SV_ERR_TOKEN;
  if (y == -2 || __ballot(!in.pg)) err |= SV_ERR_INTERNAL;
  if (STOCH && has) {
    if (P.p_target) P.p_target[b * k + lane] = err ? NAN : in.pr.pt;
    if (P.p_draft) P.p_draft[b * k + lane] = err ? NAN : in.pr.pd;
  }
  int32_t* out = P.out_tokens + b * (k + 1);
  for (int64_t j = lane; j <= k; j += WAVE) {
    int v = -1;
    if (!err) v = (j < L) ? in.x : (j == L ? y : -1);
    out[j] = v;
  }
  if (P.commit) {
    // the commit of spec_commit_linear, applied by the same wave
    const int len = P.seq_len[b];   // every lane reads it before lane 0 updates it
    const bool full = !err && P.history && (len < 0 || (int64_t)len + L + 1 > P.capacity);
    const bool ok = !err && !full;
    if (full) err |= SV_ERR_CAPACITY;
    if (lane <= k) {
      const int64_t j = lane;
      if (ok && j <= L && P.history) P.history[b * P.capacity + len + j] = (j < L) ? in.x : y;
      if (P.shifted) P.shifted[b * (k + 1) + j] = !ok ? -1 : ((j == L || j == k) ? y : in.x);
    }
    if (lane == 0) {
      if (ok) P.seq_len[b] = len + L + 1;
      if (P.next_token) P.next_token[b] = ok ? y : -1;
    }
  }
  if (lane == 0) {
    P.accept_len[b] = (err & ~SV_ERR_CAPACITY) ? -1 : L;
    if (P.err_flags) P.err_flags[b] = err;
  }
}

template <int DT, bool STOCH>
__device__ __forceinline__ void linear_emit(const LinearParams& P, int64_t b, int known_y) {
  const EmitIn in = emit_load<DT, STOCH>(P, b, known_y != TOKEN_UNKNOWN);
  emit_store<DT, STOCH>(P, b, in, known_y);
  if constexpr (STOCH) emit_clear(P, b, known_y == TOKEN_UNKNOWN);
}

// Events a wave counts when it is done: n of sequence b (n = 0: none), the final
// token among them if `token`. Every role returns its events to the kernel body,
// which counts them at one place. An event that set error bits of its sequence
// adds EV_ERR as well, so the count also tells the last event whether the error
// word needs reading.
struct Ev {
  int64_t b;
  uint32_t n;
  bool token;
  int y;
};
constexpr uint32_t EV_ERR = 1u << 16, EV_COUNT = EV_ERR - 1u;

// Counts n events of sequence b (k pair combines, target row k and, where no
// residual wave draws it, the final token); the event that completes the count
// writes the outputs. The token event carries the token: if it is not the last
// event, the token goes to the token record for the wave that will be. (A
// correction token drawn by a residual wave is not counted: that wave emits, see
// others_counted.)
template <int DT, bool STOCH>
__device__ __forceinline__ void linear_event(const LinearParams& P, int64_t b, bool token, int y, uint32_t n) {
  const uint32_t total = (uint32_t)P.EV;
  uint32_t old = 0;
  if (lane_id() == 0) old = counter_add(P.fin + b * CSTRIDE, n);
  old = bcast(old);
  if ((old & EV_COUNT) + (n & EV_COUNT) != total) {
    if (token && lane_id() == 0) {
      Token t;
      t.y = y;
      put_rec(P.tok + b, t, P.tag);
    }
    return;
  }
  linear_emit<DT, STOCH>(P, b, token ? y : TOKEN_UNKNOWN);
}

// The emission's reads that do not depend on the sequence's other events, issued
// by a wave that draws the final token together with its event's count, before its
// draw, so that their round trip overlaps the draw: the drafts, and one read of
// each position's probability record (polled for again if it was not there yet).
struct EmitPre {
  int x;
  uint64_t w[PROB_WORDS];
};
__device__ __forceinline__ EmitPre emit_prefetch(const LinearParams& P, int64_t b) {
  const int lane = lane_id();
  EmitPre e;
  e.x = 0;
#pragma unroll
  for (int i = 0; i < PROB_WORDS; ++i) e.w[i] = 0;
  if (lane < P.k) {
    e.x = P.tokens[b * P.k + lane];
#pragma unroll
    for (int i = 0; i < PROB_WORDS; ++i)
      e.w[i] = __hip_atomic_load(P.prob + (b * P.k + lane) * PROB_WORDS + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return e;
}

// The emission of sequence b by the wave that drew its final token y with L
// settled (a rejection at L < k, or every draft accepted, L = k), once the event
// count `fo` (the other events', with their EV_ERR) shows every other event in: L
// needs no read of the state word, and the error word is read only if an event set
// error bits. `pre` must come from emit_prefetch (its drafts are used as they are).
template <int DT>
__device__ __forceinline__ void emit_drawn(const LinearParams& P, int64_t b, int L, int y, const EmitPre& pre,
                                           uint32_t fo) {
  const int lane = lane_id();
  const int64_t k = P.k;
  EmitIn in;
  in.s = L < k ? 1ull << (32 + L) : 0ull;   // the rejected position, if any
  in.ew = 0;
  if (lane == 1 && (fo & ~EV_COUNT) != 0u)
    in.ew = __hip_atomic_load(P.errw + b * CSTRIDE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  in.t.y = y;
  in.tg = true;
  in.pg = true;
  in.x = pre.x;
  in.pr.pt = in.pr.pd = NAN;
  if (lane < k) {
    uint64_t* pr = P.prob + (b * k + lane) * PROB_WORDS;
    bool here = true;
    uint32_t w[PROB_WORDS];
#pragma unroll
    for (int i = 0; i < PROB_WORDS; ++i) {
      here = here && (uint32_t)(pre.w[i] >> 32) == P.tag;
      w[i] = (uint32_t)pre.w[i];
    }
    if (here) __builtin_memcpy(&in.pr, w, sizeof(Probs));
    else in.pg = get_rec(pr, in.pr, P.tag);
  }
  emit_store<DT, true>(P, b, in, y);
  emit_clear(P, b, false);
}

// Greedy finish of sequence b: polls the chunk records of its k+1 target rows
// until every one carries the call's tag (greedy records are few, so no counter). Lane r holds the argmax of target row r (rows read two at a time); the
// first position whose draft is not that argmax is L,
// and the target's token is the argmax of row L. The sequence's outputs are
// written here, with the same rules as the stochastic emission.
template <int DT>
__device__ __forceinline__ void greedy_finish(const LinearParams& P, int64_t b) {
  const int lane = lane_id();
  const int64_t k = P.k;
  const int R = (int)k + 1;
  // the drafts, read before the records: a read issued after the records' clearing
  // stores would wait for them (a wait for a load also waits for every store before it)
  const bool has = lane < k;
  const int xk = has ? P.tokens[b * k + lane] : 0;
  bool ok = true;
  int am = -1;
#pragma unroll 1
  for (int r0 = 0; r0 < R; r0 += 2) {
    // two rows at a time, lane l reading chunks l + 64 t of each
    uint64_t w[2][MAX_ROUNDS][2];
    bool got = false;
    WaitClock clk;
    for (bool go = true; go && !got;) {
      bool mine = true;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int t = 0; t < MAX_ROUNDS; ++t) {
          const int c = t * WAVE + lane;
          w[j][t][0] = tagged(__float_as_uint(-INFINITY), P.tag);
          w[j][t][1] = tagged((uint32_t)INT_SENTINEL, P.tag);
          if (t * WAVE < P.C && r0 + j < R && c < P.C) {
            const uint64_t* p = P.seg + (row_q<false>(P, b, r0 + j, 0) * P.C + c) * P.RW;
            w[j][t][0] = seg_load(p);
            w[j][t][1] = seg_load(p + 1);
          }
          mine = mine && (uint32_t)(w[j][t][0] >> 32) == P.tag && (uint32_t)(w[j][t][1] >> 32) == P.tag;
        }
      }
      got = __ballot(!mine) == 0ull;
      if (!got) {
        go = clk.more();
        __builtin_amdgcn_s_sleep(1);   // (longer pauses measured slower: the records arrive at the stream's end)
      }
    }
    ok = ok && got;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float m = -INFINITY;
      int idx = INT_SENTINEL;
#pragma unroll
      for (int t = 0; t < MAX_ROUNDS; ++t) {
        if (t * WAVE >= P.C) break;
        const int c = t * WAVE + lane;
        if (r0 + j < R && c < P.C) {
          uint64_t* p = P.seg + (row_q<false>(P, b, r0 + j, 0) * P.C + c) * P.RW;
          store_zero(p);
          store_zero(p + 1);
        }
        argmax_combine(m, idx, __uint_as_float((uint32_t)w[j][t][0]), (int)(uint32_t)w[j][t][1]);
      }
      wave_argmax(m, idx);
      if (lane == r0 + j) am = (m > -INFINITY && idx != INT_SENTINEL) ? idx : -1;
    }
  }
  EmitIn in;
  in.x = xk;
  in.ew = __ballot(lane < R && am < 0) ? (uint32_t)SV_ERR_ROW : 0u;
  const unsigned long long miss = __ballot(has && in.x != am);
  const int L = miss ? first_lane(miss) : (int)k;
  in.s = L < k ? (1ull << (32 + L)) : 0ull;
  in.t.y = ok ? -1 : -2;    // -2: a wait timed out (SV_ERR_INTERNAL)
  in.tg = true;
  in.pg = true;
  in.pr.pt = in.pr.pd = NAN;
  const int y = ok ? __shfl(am, L) : -2;
  emit_store<DT, false>(P, b, in, y);
}

// Queued launches (more residual waves than can wait on the GPU at once) place
// each decision in a slot, in the order the decisions are made: a rejection takes
// the next slot from the front, a sequence with every draft accepted the next one
// from the back. Their residual waves run in slot order (the first slots' before
// target row k streams, the others last in the launch), so the waves of rejecting
// sequences start first and the back slots' waves, which have nothing to draw,
// start last. Lane 0 takes the slot; publish_decision turns
// the value returned into the slot.
__device__ __forceinline__ uint64_t take_slot(const LinearParams& P, bool accepted) {
  return __hip_atomic_fetch_add(P.slots, accepted ? (1ull << 32) : 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The decision of sequence b, written once for each of its residual waves (each
// polls a copy of its own: one line polled by every residual wave of a sequence
// serialises the polls) at the sequence's own place, or at its slot in a queued
// launch (`taken`: lane 0's take_slot value). d must be the same in every lane.
__device__ __forceinline__ void publish_decision(const LinearParams& P, int64_t b, Decision d, uint64_t taken) {
  const int lane = lane_id();
  int64_t slot = b;
  if (P.queue) {
    taken = bcast(taken);
    const int64_t nf = (int64_t)(uint32_t)taken, nb = (int64_t)(taken >> 32);
    if (nf + nb >= P.B) return;   // more decisions than sequences: cannot happen, each is decided once
    if (lane == 0 && nf + nb + 1 == P.B) counter_reset(P.slots);   // the last slot: zero for the next call
    slot = d.kind == 0 ? P.B - 1 - nb : nf;
  }
  d.b = (int32_t)b;
  uint32_t w[DEC_WORDS];
  __builtin_memcpy(w, &d, sizeof(Decision));
  uint64_t* dst = P.dec + slot * P.CG * DEC_WORDS;   // CG copies of DEC_WORDS words
  const int n = P.CG * DEC_WORDS;
  for (int e0 = 0; e0 < n; e0 += WAVE) {
    const int e = e0 + lane;
    const int word = e % DEC_WORDS;
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < DEC_WORDS; ++i) if (word == i) v = w[i];
    if (e < n) __hip_atomic_store(dst + e, ((uint64_t)P.tag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Called after the state update old -> now of sequence b by the pair combine of
// position mi (whose statistics are `mine`). If this update settles L < k, hand
// rows t_L, d_L to the residual waves; if it settles L = k (every draft accepted
// and the bonus drawn), the bonus token is final: return true with it in y_out,
// for the caller to count with its own event.
template <int DT>
__device__ __forceinline__ bool linear_settle(const LinearParams& P, int64_t b, uint64_t old, uint64_t now,
                                              int64_t mi, const PairStat& mine, bool published, int& y_out) {
  const int k = (int)P.k;
  const int Ln = settled_L(now, k);
  if (Ln < 0 || settled_L(old, k) >= 0) return false;
  if (Ln < k) {
    if (!published) {
      PairStat ps = mine;
      bool got = true;
      if (Ln != mi) {
        if (lane_id() == 0) got = get_rec(P.pst + (b * k + Ln) * PST_WORDS, ps, P.tag);
        got = bcast((int)got) != 0;
        ps.Zt = bcast(ps.Zt);
        ps.Zd = bcast(ps.Zd);
        ps.Mt = bcast(ps.Mt);
        ps.Md = bcast(ps.Md);
        ps.okt = bcast(ps.okt);
        ps.okd = bcast(ps.okd);
      }
      Decision d;
      d.L = (int16_t)Ln;
      d.kind = (got && ps.okt && ps.okd) ? 1 : 2;
      d.Mt = ps.Mt;
      d.Md = ps.Md;
      d.Zt = ps.Zt;
      d.Zd = ps.Zd;
      uint64_t taken = 0;
      if (P.queue && lane_id() == 0) taken = take_slot(P, false);
      publish_decision(P, b, d, taken);
    }
    return false;   // the residual waves draw the token
  }
  int y = 0;
  if (lane_id() == 0) {
    RowStat rk;
    const bool got = get_rec(P.rks + b * ROW_WORDS, rk, P.tag);
    y = !got ? -2 : (rk.ok != 1 ? -1 : rk.y);
  }
  y_out = bcast(y);
  return true;
}

// Stochastic, position i < k of sequence b: combines rows t_i and d_i once all of
// their segments are in, and runs the acceptance test u_i < p_t,i(x_i) / p_d,i(x_i).
template <int DT>
__device__ __forceinline__ Ev pair_finish(const LinearParams& P, int64_t b, int64_t i) {
  const int lane = lane_id();
  const int64_t k = P.k, V = P.V;
  const int x = P.tokens[b * k + i];
  const int64_t qt = row_q<true>(P, b, i, 0);
  // the state as it was when the last records arrived: if every earlier position
  // is already accepted, a rejection here settles L = i without the state
  // update's round trip
  uint64_t se = 0;
  RowParts rp[2];
  const bool got = read_rows<2>(P, qt, rp, i > 0 ? P.state + b * SSTRIDE : nullptr, &se);
  double wl[MAX_ROUNDS];
  const RowSums st = row_sums<true, false>(rp[0], P.c0, wl, P.C);
  const RowSums sd = row_sums<true, false>(rp[1], P.c0, wl, P.C);
  const RowParts& rt = rp[0];
  const RowParts& rd = rp[1];
  const bool okt = got && st.M > -INFINITY && __builtin_isfinite(st.Z) && st.Z > 0.0;
  const bool okd = got && sd.M > -INFINITY && __builtin_isfinite(sd.Z) && sd.Z > 0.0;
  const bool xok = x >= 0 && x < V;
  double pxt = NAN, pxd = NAN;
  if (okt && xok && rt.xin) pxt = exp2(((double)rt.xv - (double)st.M) * (double)P.c0) / st.Z;
  if (okd && xok && rd.xin) pxd = exp2(((double)rd.xv - (double)sd.M) * (double)P.c0) / sd.Z;
  // Both probabilities as fp32: the ratio keeps about 1e-7 relative. Below the
  // smallest normal fp32 (or at zero) that no longer holds, and the test takes both
  // in fp64.
  const float ft = okt ? (float)pxt : NAN, fd = okd ? (float)pxd : NAN;
  double pt = (double)ft, pd = (double)fd;
  if (ft < FLT_MIN || fd < FLT_MIN) {   // NaN (an unusable row) compares false
    pt = okt ? pxt : (double)NAN;
    pd = okd ? pxd : (double)NAN;
  }
  double qr;
  if (pd > 0.0) qr = pt / pd;
  else qr = (pt > 0.0) ? INFINITY : NAN;
  const bool ok = !isnan(pt) && !isnan(pd);   // an unusable row rejects
  const bool acc = ok && (double)P.uniforms[b * (k + 1) + i] < qr;   // NaN ratio rejects
  const uint64_t bits = (1ull << i) | (acc ? 0ull : (1ull << (32 + i)));
  PairStat ps;
  ps.Zt = st.Z;
  ps.Zd = sd.Z;
  ps.Mt = st.M;
  ps.Md = sd.M;
  ps.okt = okt;
  ps.okd = okd;
  se = bcast(se);
  const uint64_t before = (1ull << i) - 1;
  // if so, this wave's state update is the one that settles L = i (see linear_settle)
  const bool early = !acc && (se & before) == before && ((se >> 32) & before) == 0;
  Decision de;
  de.L = (int16_t)i;
  de.kind = (okt && okd) ? 1 : 2;
  de.Mt = ps.Mt;
  de.Md = ps.Md;
  de.Zt = ps.Zt;
  de.Zd = ps.Zd;
  Probs pr;
  pr.pt = (float)pt;
  pr.pd = (float)pd;
  // An early decision goes out after this position's probability record, which
  // the wave that will emit reads as soon as it has the decision (were the record
  // not there yet, that wave would poll for it again, a round trip more).
  if (early && !P.queue) {
    put_rec_wave(P.prob + (b * k + i) * PROB_WORDS, pr, P.tag);
    publish_decision(P, b, de, 0);
  }
  // Otherwise the state update first: an atomic whose result the wave waits for
  // also waits for every store the wave issued before it, and the records below
  // are read by polling, so they may land later. A queued launch's early decision
  // needs its slot first; that round trip overlaps the state update's.
  uint64_t olds = 0, taken = 0;
  if (lane == 0) {
    if (!got) error_or(P.errw + b * CSTRIDE, (uint32_t)SV_ERR_INTERNAL);
    else if (!okt || !okd) error_or(P.errw + b * CSTRIDE, (uint32_t)SV_ERR_ROW);
    olds = state_or(P.state + b * SSTRIDE, bits);
    if (early && P.queue) taken = take_slot(P, false);
  }
  if (!(early && !P.queue)) put_rec_wave(P.prob + (b * k + i) * PROB_WORDS, pr, P.tag);
  if (early && P.queue) publish_decision(P, b, de, taken);
  put_rec_wave(P.pst + (b * k + i) * PST_WORDS, ps, P.tag);
  olds = bcast(olds);
  {
    // The update that decides the last position with none rejected tells the
    // residual waves that L = k (they have nothing to draw), without waiting for
    // target row k.
    const uint64_t mk = (1ull << k) - 1, now = olds | bits;
    if ((now & mk) == mk && ((now >> 32) & mk) == 0 && (olds & mk) != mk) {
      Decision d;
      d.L = (int16_t)k;
      d.kind = 0;
      d.Mt = d.Md = 0.0f;
      d.Zt = d.Zd = 0.0;
      uint64_t tk = 0;
      if (P.queue && lane == 0) tk = take_slot(P, true);
      publish_decision(P, b, d, tk);
    }
  }
  const uint32_t ef = (!got || !okt || !okd) ? EV_ERR : 0u;   // it set error bits
  int y = 0;
  if (linear_settle<DT>(P, b, olds, olds | bits, i, ps, early, y)) {
    // L = k and the bonus token is final: this position's event and the token's,
    // counted here with the emission's reads alongside
    uint32_t fo = 0;
    if (lane == 0) fo = counter_add(P.fin + b * CSTRIDE, 2u | ef);
    const EmitPre pre = emit_prefetch(P, b);
    fo = bcast(fo);
    if ((fo & EV_COUNT) + 2 == (uint32_t)P.EV) {
      emit_drawn<DT>(P, b, (int)k, y, pre, fo | ef);
    } else if (lane == 0) {
      Token t;
      t.y = y;
      put_rec(P.tok + b, t, P.tag);
    }
    return Ev{0, 0u, false, 0};
  }
  return Ev{b, 1u | ef, false, 0};
}

// Stochastic, target row k of sequence b (the row after the last draft): combined
// once all of its segments are in; draws the bonus token from p_t,k unless an
// earlier position is already rejected.
template <int DT>
__device__ __forceinline__ Ev rowk_finish(const LinearParams& P, int64_t b) {
  const int lane = lane_id();
  const int64_t k = P.k, V = P.V;
  uint64_t sn = 0;   // the state, read with the records
  RowParts rpa[1];
  const bool got = read_rows<1>(P, row_q<true>(P, b, k, 0), rpa, P.state + b * SSTRIDE, &sn);
  const RowParts& rp = rpa[0];
  double wl[MAX_ROUNDS];
  const RowSums rs = row_sums<true, false>(rp, P.c0, wl, P.C);
  RowStat st;
  st.Z = rs.Z;
  st.M = rs.M;
  st.argmax = rs.argmax;
  st.px = NAN;
  st.y = -1;
  st.ok = !got ? -1 : ((rs.M > -INFINITY && __builtin_isfinite(rs.Z) && rs.Z > 0.0) ? 1 : 0);
  sn = bcast(sn);
  // The state update goes out before the draw, so that its round trip overlaps it
  // (a wave that settles L = k from the state word polls for this row's record,
  // which follows the draw).
  uint64_t olds = 0;
  if (lane == 0) {
    if (st.ok != 1) error_or(P.errw + b * CSTRIDE, (uint32_t)(st.ok < 0 ? SV_ERR_INTERNAL : SV_ERR_ROW));
    olds = state_or(P.state + b * SSTRIDE, BONUS_BIT);   // before the record (see pair_finish)
  }
  if (st.ok == 1 && settled_L(sn, (int)k) < 0)
    st.y = softmax_draw<DT>(row_ptr<DT, true>(P, b, k, 0), V, P.C, P.c0, P.uniforms[b * (k + 1) + k], rp, rs, wl);
  put_rec_wave(P.rks + b * ROW_WORDS, st, P.tag);
  olds = bcast(olds);
  const int Ln = settled_L(olds | BONUS_BIT, (int)k);
  const uint32_t ef = st.ok != 1 ? EV_ERR : 0u;   // it set error bits
  if (Ln == (int)k && settled_L(olds, (int)k) < 0) {
    // the bonus token is final: this row's event and the token's, counted here,
    // with the emission's reads alongside
    uint32_t fo = 0;
    if (lane == 0) fo = counter_add(P.fin + b * CSTRIDE, 2u | ef);
    const EmitPre pre = emit_prefetch(P, b);
    fo = bcast(fo);
    if ((fo & EV_COUNT) + 2 == (uint32_t)P.EV) {
      emit_drawn<DT>(P, b, (int)k, st.y, pre, fo | ef);
    } else if (lane == 0) {
      Token t;
      t.y = st.y;
      put_rec(P.tok + b, t, P.tag);
    }
    return Ev{0, 0u, false, 0};
  }
  return Ev{b, 1u | ef, false, 0};
}

// Streaming wave of chunk c of row q: the chunk's partial goes out as its record.
// Nothing here waits for another wave.
template <int DT, bool STOCH>
__device__ __forceinline__ void linear_chunk_wave(const LinearParams& P, uint32_t q32, uint32_t c32) {
  const int lane = lane_id();
  int64_t b, i;
  int which;
  row_of_q<STOCH>(P, q32, b, i, which);
  const char* row = row_ptr<DT, STOCH>(P, b, i, which);
  const int64_t x = (STOCH && i < P.k) ? (int64_t)P.tokens[b * P.k + i] : -1;
  const Partial p = chunk_partial<DT, STOCH, !STOCH>(row, P.V, c32, P.c0, x);
  uint64_t* rec = P.seg + ((int64_t)q32 * P.C + c32) * P.RW;
  if constexpr (STOCH) {
    const uint64_t sb = (uint64_t)__double_as_longlong(p.s);
    const uint32_t word = lane == 0 ? __float_as_uint(p.m)
                        : lane == 1 ? (uint32_t)sb
                        : lane == 2 ? (uint32_t)(sb >> 32)
                        : (p.xin ? __float_as_uint(p.xv) : NOT_HELD);
    if (lane < 4) seg_store(rec + lane, tagged(word, P.tag));
  } else {
    if (lane < 2) seg_store(rec + lane, tagged(lane == 0 ? __float_as_uint(p.m) : (uint32_t)p.idx, P.tag));
  }
}

// The event count of sequence b once its other events (k pair decisions and target
// row k) have all counted, for the wave that drew its correction token: that wave
// counts no event of its own and is always the one that emits (no other event's
// count reaches the total). `snap` is a read of the count taken earlier; polled
// again only if it was short. A wait that gives up sets SV_ERR_INTERNAL and
// returns with EV_ERR, so that the emission reads the error word.
__device__ __forceinline__ uint32_t others_counted(const LinearParams& P, int64_t b, uint32_t snap) {
  const uint32_t want = (uint32_t)P.EV - 1u;
  if ((snap & EV_COUNT) == want) return snap;
  uint32_t v = snap;
  if (lane_id() == 0) {
    WaitClock clk;
    for (;;) {
      v = __hip_atomic_load(P.fin + b * CSTRIDE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((v & EV_COUNT) == want) break;
      if (!clk.more()) {
        error_or(P.errw + b * CSTRIDE, (uint32_t)SV_ERR_INTERNAL);
        v |= EV_ERR;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  return bcast(v);
}

// Residual wave (b, g), dispatched after the streaming waves of every row a
// decision depends on: waits for the decision of sequence b (in a queued launch:
// the decision in slot b, which names its sequence); if a draft was rejected, sums
// the residual max(0, p_t,L - p_d,L) over part g (half a chunk) of rows t_L, d_L.
// The sequence's last residual wave to count picks the part that holds u*S.
// Without hold mode it reloads that part and scans it. In hold mode (a launch
// whose residual waves can all be resident at once, so that none waits for a wave
// that cannot start) every residual wave keeps its part and its unit sums and
// waits for the last one's verdict; the wave holding the picked part scans it from
// its registers. The wave that draws writes the outputs (see others_counted): a
// token event counted ahead of the draw let another event's wave become the last
// one, which then waited for the token record, a round trip more (about half the
// rejecting sequences at C2).
template <int DT>
__device__ __forceinline__ Ev linear_residual_wave(const LinearParams& P, int64_t b, int64_t g) {
  const int lane = lane_id();
  const uint32_t CG = (uint32_t)P.CG;   // residual waves per sequence
  const int64_t k = P.k;
  Decision d;
  d.L = 0;
  d.kind = 2;
  d.b = (int32_t)b;
  d.Mt = d.Md = 0.0f;
  d.Zt = d.Zd = 0.0;
  uint64_t* dr = P.dec + (b * P.CG + g) * DEC_WORDS;   // this wave's copy of the decision
  if (!poll_rec(dr, d, P.tag)) d.kind = 3;   // 3: the decision never arrived
  // The records this wave read are cleared for the next call on its way out: a
  // wait for a load (or a returning atomic) also waits for every store the wave
  // issued before it, and these device-scope stores take about a microsecond.
  const auto done = [&]() {
    if (lane == 0) clear_rec<Decision>(dr);
  };
  if (P.queue) {
    // the slot's sequence; a slot whose decision never arrived names none
    if (d.kind == 3 || d.b < 0 || d.b >= P.B) {
      done();
      return Ev{0, 0u, false, 0};
    }
    b = d.b;
  }
  const char* trow = row_ptr<DT, true>(P, b, d.kind == 1 ? d.L : 0, 0);
  const char* drow = row_ptr<DT, true>(P, b, d.kind == 1 ? d.L : 0, 1);
  const ResidW rw = make_residw(d, P.c0);
  // No draft rejected: nothing to draw here (the bonus token is target row k's), so
  // no count either; each residual wave clears its own copy of the decision.
  if (d.kind == 0) {
    done();
    return Ev{0, 0u, false, 0};
  }
  // Counted before the sums: the count's round trip overlaps this wave's loads. The
  // last to count draws; it reads the others' records with polling reads, which
  // wait for any that are not written yet.
  uint32_t old = 0;
  if (lane == 0) old = counter_add(P.res_cnt + b * CSTRIDE, 1u);
  // part g of the sequence's rows: chunk g / RH, half g % RH
  const int64_t u0 = (g / RH) * CHUNK_UNITS + (g % RH) * (HU * WAVE);
  RawN<HU> rt, rd;
  Chunk kg;
  float us[HU];
  if (d.kind == 1) {
    kg = load_units<DT, HU>(trow, P.V, u0, rt);
    load_units<DT, HU>(drow, P.V, u0, rd);
    ResPart r;
    r.s = residual_raw_sum<DT>(rt, rd, rw, us);
    put_rec_wave(P.res + (b * P.CG + g) * RES_WORDS, r, P.tag);
  }
  old = bcast(old);
  const float u = P.uniforms[b * (k + 1) + k];
  if (old + 1 != CG) {
    if (!(P.hold && d.kind == 1)) {
      done();
      return Ev{0, 0u, false, 0};
    }
    // hold mode: wait for the verdict on this part
    uint64_t* vr = P.verd + (b * P.CG + g) * VERD_WORDS;
    Verdict v;
    v.kind = 0;
    v.fo = 0;
    v.th = 0.0;
    const bool got = poll_rec(vr, v, P.tag);
    if (!got || v.kind == 0) {
      if (lane == 0) clear_rec<Verdict>(vr);
      done();
      return Ev{0, 0u, false, 0};
    }
    // this wave emits: the emission's reads go out before the scan, so that their
    // round trip overlaps it
    const EmitPre pre = emit_prefetch(P, b);
    ResidW rx = rw;
    int yh;
    if (v.kind == 2) {
      // no residual mass: p_t,L's weights (the draft's zeroed, taken from row t_L)
      rx.mc0d = rx.mc0t;
      rx.izd = 0.0f;
      chunk_unit_sums<DT, true>(rt, rt, rx, us);
      yh = (int)chunk_invcdf_us<DT, true>(kg, rt, rt, us, v.th, rx);
    } else {
      yh = (int)chunk_invcdf_us<DT, true>(kg, rt, rd, us, v.th, rx);
    }
    const uint32_t fo = others_counted(P, b, v.fo);
    emit_drawn<DT>(P, b, d.L, yh, pre, fo);
    if (lane == 0) clear_rec<Verdict>(vr);
    done();
    return Ev{0, 0u, false, 0};
  }
  // last residual wave of the sequence: draw the correction token; the part
  // records and the counter are cleared on the way out
  const auto done_last = [&]() {
    if (lane == 0) counter_reset(P.res_cnt + b * CSTRIDE);
    for (int cc = lane; cc < (int)CG; cc += WAVE) clear_rec<ResPart>(P.res + (b * P.CG + cc) * RES_WORDS);
    done();
  };
  int y = (d.kind == 3) ? -2 : -1;
  if (d.kind != 1) {   // the final token (no draw: a data error or a timed-out wait)
    done_last();
    return Ev{b, 1u, true, y};
  }
  // A read of the other events' count and the emission's reads go out with the
  // reads of the residual sums (in hold mode the count is passed on in the
  // verdicts). Whichever wave draws the token writes the outputs, once every other
  // event has counted (see others_counted).
  uint32_t fo = 0;
  if (lane == 0) fo = __hip_atomic_load(P.fin + b * CSTRIDE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const EmitPre pre = emit_prefetch(P, b);
  constexpr int RR = RH * MAX_ROUNDS;   // rounds of 64 parts
  double wl[RR];
  bool ok = true;
#pragma unroll
  for (int t = 0; t < RR; ++t) {
    wl[t] = 0.0;
    if (t * WAVE >= (int)CG) continue;
    const int cc = t * WAVE + lane;
    if (cc < (int)CG) {
      ResPart r;
      uint64_t* rec = P.res + (b * P.CG + cc) * RES_WORDS;
      const bool gr = get_rec(rec, r, P.tag);
      ok = ok && gr;
      wl[t] = gr ? r.s : 0.0;
    }
  }
  fo = bcast(fo);
  ChunkPick pk;
  pk.c = -1;
  ResidW rx = rw;
  const char* dx = drow;
  bool zero = false;   // no residual mass: the draw comes from p_t,L
  const bool rec_ok = __ballot(!ok) == 0ull;
  if (!rec_ok) {
    y = -2;
  } else {
    // The draw from the residual. With no residual mass (the rows agree up to
    // rounding) it is taken from p_t,L instead: the same pick and scan with the
    // draft's weights zeroed (and taken from row t_L, so that they stay finite),
    // over chunk sums formed here.
    pk = pick_chunk((int)CG, (double)u, wl);
    if (pk.c < 0 && pk.total == 0.0) {
      zero = true;
      rx.mc0d = rx.mc0t;
      rx.izd = 0.0f;
      dx = trow;
#pragma unroll
      for (int t = 0; t < RR; ++t) wl[t] = 0.0;
      // (this wave's own registers serve as the buffer)
#pragma unroll 1
      for (int c = 0; c < (int)CG; ++c) {
        load_units<DT, HU>(trow, P.V, (c / RH) * CHUNK_UNITS + (c % RH) * (HU * WAVE), rt);
        const double sc = residual_raw_sum<DT>(rt, rt, rx, us);
#pragma unroll
        for (int t = 0; t < RR; ++t)
          if (t * WAVE + lane == c) wl[t] = sc;
      }
      pk = pick_chunk((int)CG, (double)u, wl);
    }
  }
  const double th = pk.fallback ? (double)INFINITY : pk.theta - pk.before;
  if (P.hold) {
    // every other residual wave of the sequence waits for its verdict (one store
    // instruction: lane c writes part c's kind, the picked part's record whole)
    const int pc = pk.c;
    for (int c0 = 0; c0 < (int)CG; c0 += WAVE) {
      const int c = c0 + lane;
      if (c < (int)CG && c != g) {
        Verdict v;
        v.kind = c == pc ? (zero ? 2 : 1) : 0;
        v.fo = fo;
        v.th = th;
        put_rec(P.verd + (b * P.CG + c) * VERD_WORDS, v, P.tag);
      }
    }
    if (pc >= 0 && pc != g) {   // the holder draws and emits
      done_last();
      return Ev{0, 0u, false, 0};
    }
    // nothing to draw from (pc < 0: the token is -1, or -2 after a timed-out read),
    // or the pick is this wave's own chunk, whose registers were not kept: the
    // reload below serves
  }
  // the picked part, reloaded into this wave's own registers
  if (pk.c >= 0) {
    const int64_t pu = (pk.c / RH) * CHUNK_UNITS + (pk.c % RH) * (HU * WAVE);
    kg = load_units<DT, HU>(trow, P.V, pu, rt);
    load_units<DT, HU>(dx, P.V, pu, rd);
  }
  if (pk.c >= 0) y = (int)chunk_invcdf<DT, true>(kg, rt, rd, th, rx);
  fo = others_counted(P, b, fo);
  emit_drawn<DT>(P, b, d.L, y, pre, fo);
  done_last();
  return Ev{0, 0u, false, 0};
}

// Wave roles of a linear launch, in dispatch order. Greedy: the chunk waves of
// every row (rows of position 0 of every sequence, then position 1, ...), then one
// finishing wave per sequence. Stochastic: for each position i < k and each
// sequence, the chunk waves of its target and draft rows (chunk by chunk,
// alternating) and the wave that finishes the pair; then for each sequence the
// chunk waves of its target row k, the wave that finishes that row, and (hold
// mode) its residual waves, RH per chunk. A queued launch has its residual waves
// last instead, in slot order (see take_slot). Every wave that waits follows the
// waves it waits for. Each finishing wave comes right after its own rows, so that
// decisions are made while later rows still stream, and residual waves come after
// all pairs of their sequence: most of them find their decision made and either
// draw at once (overlapping the remaining stream) or, if nothing was rejected, end
// at once.
enum RoleKind { ROLE_IDLE = 0, ROLE_STREAM, ROLE_RESID, ROLE_PAIR, ROLE_ROWK, ROLE_GREEDY };
struct Role {
  int kind;
  uint32_t q, b, c;   // stream: row q, chunk c; residual: sequence (queued: slot) b, part c; finishers: sequence b, position c
};

template <bool STOCH>
__device__ __forceinline__ Role linear_role(const LinearParams& P, uint32_t w) {
  Role r;
  r.kind = ROLE_IDLE;
  r.q = r.b = r.c = 0;
  const uint32_t NS = (uint32_t)P.C, B = (uint32_t)P.B;
  if constexpr (!STOCH) {
    const uint32_t ns = (uint32_t)(P.k + 1) * B * NS;
    if (w < ns) {
      r.q = w / NS;
      r.c = w - r.q * NS;
      r.kind = ROLE_STREAM;
    } else {
      r.b = w - ns;
      r.kind = ROLE_GREEDY;
    }
  } else {
    if (w < P.tk0) {
      // position blocks of B pair blocks of 2C + 1 waves
      const uint32_t QP = 2 * NS + 1;
      const uint32_t blk = w / QP, e = w - blk * QP;
      const uint32_t pos = blk / B;
      r.b = blk - pos * B;
      if (e < 2 * NS) {
        r.q = pos * 2 * B + 2 * r.b + (e & 1u);
        r.c = e >> 1;
        r.kind = ROLE_STREAM;
      } else {
        r.c = pos;
        r.kind = ROLE_PAIR;
      }
    } else {
      // the CG residual waves of `early` sequences (hold mode: all of them) or
      // decision slots (queued), then the sequence blocks (the C chunk waves of
      // target row k and its finisher), then a queued launch's other slots
      const uint32_t CG = (uint32_t)P.CG;
      const uint32_t Q = NS + 1;
      const uint32_t E = P.early * CG;
      uint32_t v = w - P.tk0;
      if (v < E) {
        r.b = v / CG;
        r.c = v - r.b * CG;
        r.kind = ROLE_RESID;
        return r;
      }
      v -= E;
      if (v < B * Q) {
        r.b = v / Q;
        const uint32_t e = v - r.b * Q;
        if (e < NS) {
          r.q = (uint32_t)(2 * P.k) * B + r.b;
          r.c = e;
          r.kind = ROLE_STREAM;
        } else {
          r.kind = ROLE_ROWK;
        }
      } else {
        const uint32_t x = v - B * Q + E;   // queued: slot x / CG, part x mod CG
        r.b = x / CG;
        r.c = x - r.b * CG;
        r.kind = ROLE_RESID;
      }
    }
  }
  return r;
}

template <int DT, bool STOCH>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(3))) void linear_kernel(LinearParams args) {
  (void)args;
  const LinearParams& P = kernel_args<LinearParams>();
  const int64_t w = (int64_t)blockIdx.x * WPB + wave_in_block();
  if (w >= P.n_waves) return;
  const Role r = linear_role<STOCH>(P, (uint32_t)w);
  Ev ev{0, 0u, false, 0};
  if (r.kind == ROLE_STREAM) {
    linear_chunk_wave<DT, STOCH>(P, r.q, r.c);
  } else if constexpr (STOCH) {
    if (r.kind == ROLE_PAIR) ev = pair_finish<DT>(P, r.b, r.c);
    else if (r.kind == ROLE_ROWK) ev = rowk_finish<DT>(P, r.b);
    else if (r.kind == ROLE_RESID) ev = linear_residual_wave<DT>(P, r.b, r.c);
  } else {
    if (r.kind == ROLE_GREEDY) greedy_finish<DT>(P, r.b);
  }
  if (STOCH && ev.n) linear_event<DT, STOCH>(P, ev.b, ev.token, ev.y, ev.n);
  if constexpr (STOCH) {
    // the finishers' chunk records, cleared last
    if (r.kind == ROLE_PAIR) clear_rows<2>(P, row_q<true>(P, r.b, r.c, 0));
    else if (r.kind == ROLE_ROWK) clear_rows<1>(P, row_q<true>(P, r.b, P.k, 0));
  }
}

// ------------------------------------------------------------------ trees
struct TreeParams {
  const char* logits;
  const int32_t* parent;
  int64_t parent_stride;
  const int32_t* cand;
  const float* uniforms;
  int32_t* accept_len;
  int32_t* path_nodes;
  int32_t* out_tokens;
  int32_t* err_flags;
  uint64_t* parts;      // [B*N][C] Partial records
  uint32_t* row_cnt;    // [B*N]
  int32_t* node_y;      // [B][N] token of each node (-1 unusable row, -2 a wait timed out)
  uint64_t* yrec;       // [B][N] the same as Token records, when the stream launch walks the trees
  uint32_t* tree_cnt;   // [B]    nodes combined per tree (wave walk)
  bool wave_walk;       // trees of at most WAVE_WALK_NODES nodes, tokens known while streaming
  float* xl;            // [B][N] typical acceptance: each candidate's logit in its parent's row
  int64_t n_gather;     // typical acceptance: waves that gather xl, ahead of the streaming waves
  bool row_waves;       // one streaming wave per row (large batches), else one per (row, chunk)
  struct NodeStat* nstat;   // [B][N] typical acceptance: each node's softmax statistics
  int64_t B, N, V, max_depth;
  int C, CP;
  float c0;
  double l2eps, l2delta;   // typical acceptance: log2 of eps and delta (-inf for 0)
  uint32_t tag;
  int64_t n_stream;
};

// Typical acceptance, the gate of a node: a child's candidate v passes iff
// p(v) = exp2((x_v - M) c0) / Z > min(eps, delta * exp(-H)), with max M, normaliser
// Z = sum_v exp2((x_v - M) c0) and entropy H (nats) of softmax(row / T); in base-2
// logarithms, iff (x_v - M) c0 > G = log2(Z) + log2(min(eps, delta * exp(-H))).
// With S1 = sum_v w_v (x_v - M) c0 over the weights w_v = exp2((x_v - M) c0),
// H / ln 2 = log2(Z) - S1 / Z, so G = min(log2(Z) + log2(eps), log2(delta) + S1 / Z).
struct NodeStat {
  double G;
  float M;
  int ok;
};

// How the token of a node is chosen. Greedy: its argmax, while streaming.
// Stochastic: an inverse-CDF draw with the node's uniform, either while streaming
// at every node (EAGER: the draws overlap the stream, best for few rows) or by
// the walk at the accepted nodes only (LAZY: the only draws the result depends
// on, best for many rows).
// TYPICAL: typical acceptance, the row's statistics with its entropy for the walk.
enum TreeDraw { TD_ARGMAX = 0, TD_EAGER = 1, TD_LAZY = 2, TD_TYPICAL = 3 };
constexpr int64_t TREE_EAGER_ROWS = 4096;   // at most this many rows (B * n_nodes) draw eagerly

static_assert(RecWords<EntPartial>::N == PART_WORDS, "entropy partials use the partial records");

// Typical acceptance, streaming wave of row q, chunk c: the chunk's entropy
// partial; the row's last chunk combines them into the node's statistics.
// One wave streams all C chunks of a row, two in flight at a time, and hands each
// chunk's partial (the same in every lane) to put(c, partial): the row waves of
// large tree batches, which need neither partial records nor arrival counters.
template <int DT, class Reduce, class Put>
__device__ __forceinline__ void row_chunks(const char* row, int64_t V, int C, Reduce reduce, Put put) {
  Raw ra, rb;
  Chunk ka = load_chunk<DT>(row, V, 0, ra);
#pragma unroll 1
  for (int c = 0; c < C; c += 2) {
    Chunk kb;
    if (c + 1 < C) kb = load_chunk<DT>(row, V, c + 1, rb);
    put(c, reduce(ka, ra));
    if (c + 2 < C) ka = load_chunk<DT>(row, V, c + 2, ra);
    if (c + 1 < C) put(c + 1, reduce(kb, rb));
  }
}

// Typical acceptance: the entropy partials of row q, lane l holding chunks
// l + 64 t: from the records of its chunk waves (by the last of them; false for
// the others), or streamed by a row wave.
struct EntParts {
  float m[MAX_ROUNDS];
  double sv[MAX_ROUNDS], s1[MAX_ROUNDS];
  bool got;
};

template <int DT, bool ROWS>
__device__ __forceinline__ bool tree_typical_parts(const TreeParams& P, const char* row, int64_t q, int64_t c,
                                                   EntParts& ep) {
  const int lane = lane_id();
#pragma unroll
  for (int t = 0; t < MAX_ROUNDS; ++t) {
    ep.m[t] = -INFINITY;
    ep.sv[t] = ep.s1[t] = 0.0;
  }
  ep.got = true;
  if constexpr (ROWS) {
    row_chunks<DT>(row, P.V, P.C, [&](const Chunk&, const Raw& r) { return chunk_reduce_ent<DT>(r, P.c0); },
                   [&](int cc, const EntPartial& e) {
#pragma unroll
                     for (int t = 0; t < MAX_ROUNDS; ++t)
                       if (t * WAVE + lane == cc) {
                         ep.m[t] = e.m;
                         ep.sv[t] = e.s;
                         ep.s1[t] = e.s1;
                       }
                   });
    return true;
  } else {
  Raw r;
  load_chunk<DT>(row, P.V, c, r);
  const EntPartial p = chunk_reduce_ent<DT>(r, P.c0);
  uint32_t old = 0;
  if (lane == 0) {
    put_rec(P.parts + (q * P.C + c) * PART_WORDS, p, P.tag);
    old = counter_add(P.row_cnt + q * CSTRIDE, 1u);
  }
  if (bcast(old) + 1 != (uint32_t)P.C) return false;
  if (lane == 0) counter_reset(P.row_cnt + q * CSTRIDE);
  bool got = true;
#pragma unroll
  for (int t = 0; t < MAX_ROUNDS; ++t) {
    EntPartial e;
    e.m = -INFINITY;
    e.s = e.s1 = 0.0;
    const int cc = t * WAVE + lane;
    if (cc < P.C) {
      uint64_t* rec = P.parts + (q * P.C + cc) * PART_WORDS;
      got = get_rec(rec, e, P.tag) && got;
      clear_rec<EntPartial>(rec);
    }
    ep.m[t] = e.m;
    ep.sv[t] = e.s;
    ep.s1[t] = e.s1;
  }
  ep.got = __ballot(!got) == 0ull;
  return true;
  }
}

// Typical acceptance: the node's statistics from its entropy partials.
__device__ __forceinline__ void tree_typical_combine(const TreeParams& P, int64_t q, const EntParts& ep) {
  const int lane = lane_id();
  float M = -INFINITY;
#pragma unroll
  for (int t = 0; t < MAX_ROUNDS; ++t) M = fmaxf(M, ep.m[t]);
  M = wave_max(M);
  const double Mc0 = (double)M * (double)P.c0;
  double Z = 0.0, S1 = 0.0;
#pragma unroll
  for (int t = 0; t < MAX_ROUNDS; ++t) {
    if (ep.m[t] == -INFINITY) continue;
    // chunk weights are relative to fl32(m*c0): bring them to the row max
    const double f = pow2_neg((double)chunk_mc0(ep.m[t], P.c0) - Mc0);
    // exponents relative to the row: t_v + (fl32(m*c0) - M*c0)
    Z += ep.sv[t] * f;
    S1 += (ep.s1[t] + ((double)chunk_mc0(ep.m[t], P.c0) - Mc0) * ep.sv[t]) * f;
  }
  Z = wave_sum(Z);
  S1 = wave_sum(S1);   // sum_v w_v (x_v - M) c0
  NodeStat st;
  st.M = M;
  // log2(Z) from Z = m 2^e, m in [0.5, 1): e + log2(m), the fraction's log2 in fp32
  // (absolute error about 1e-7)
  int ez = 0;
  const double mz = frexp(Z, &ez);
  const double l2z = (double)ez + (double)__builtin_amdgcn_logf((float)mz);
  const double g1 = l2z + P.l2eps, g2 = P.l2delta + S1 / Z;
  st.G = g1 < g2 ? g1 : g2;
  const bool usable = M > -INFINITY && __builtin_isfinite(Z) && Z > 0.0 && __builtin_isfinite(S1);
  st.ok = usable ? 1 : 0;
  if (lane == 0) {
    P.nstat[q] = st;
    P.node_y[q] = !ep.got ? -2 : (usable ? 0 : -1);
  }
}

// Trees of at most WAVE_WALK_NODES nodes whose tokens are known once every row is
// combined (greedy, or stochastic with every node drawn while streaming) are
// walked by the wave that combines the tree's last node, in registers: lane l
// holds nodes l + 64 s, and a node's parent, token or match flag is fetched
// across lanes. The result is the one the walk launch computes.
constexpr int WW_SLOTS = 4;
constexpr int64_t WAVE_WALK_NODES = WW_SLOTS * WAVE;

__device__ __forceinline__ int wave_or_int(int v) {
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) v |= __shfl_xor(v, o);
  return v;
}

// The wave that combined the tree's last node walks it. Once the node tokens are
// in, it clears the token records, the tree's counter and (q >= 0) the partials of
// its own row q for the next call: the walk that follows waits for no memory, so
// these stores complete while it runs.
__device__ __forceinline__ void tree_wave_walk(const TreeParams& P, int64_t b, int64_t q) {
  const int lane = lane_id();
  const int N = (int)P.N;
  const int32_t* par = P.parent + b * P.parent_stride;
  const int32_t* cand = P.cand + b * N;
  uint64_t* yr = P.yrec + b * N;
  int pv[WW_SLOTS], cv[WW_SLOTS], yv[WW_SLOTS], st[WW_SLOTS];
  int err = 0;
#pragma unroll
  for (int s = 0; s < WW_SLOTS; ++s) {
    const int i = s * WAVE + lane;
    pv[s] = -1;
    cv[s] = 0;
    yv[s] = 0;
    if (i < N) {
      pv[s] = par[i];
      cv[s] = cand[i];
    }
  }
  // every slot's token polled in the same round trip
  static_assert(RecWords<Token>::N == 1, "one word per token record");
  {
    bool have[WW_SLOTS];
#pragma unroll
    for (int s = 0; s < WW_SLOTS; ++s) have[s] = s * WAVE + lane >= N;
    WaitClock clk;
    for (;;) {
      bool all = true;
#pragma unroll
      for (int s = 0; s < WW_SLOTS; ++s) {
        if (!have[s]) {
          const uint64_t x = __hip_atomic_load(yr + s * WAVE + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((uint32_t)(x >> 32) == P.tag) {
            yv[s] = (int)(uint32_t)x;
            have[s] = true;
          } else {
            all = false;
          }
        }
      }
      if (__ballot(!all) == 0ull) break;
      if (!clk.more()) {
#pragma unroll
        for (int s = 0; s < WW_SLOTS; ++s)
          if (!have[s]) yv[s] = -2;   // the wait gave up
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
#pragma unroll
  for (int s = 0; s < WW_SLOTS; ++s) {
    const int i = s * WAVE + lane;
    if (i < N) clear_rec<Token>(yr + i);
  }
  if (q >= 0) clear_parts<Partial>(P.parts + q * P.C * PART_WORDS, P.C, P.row_cnt + q * CSTRIDE);
  if (lane == 0) counter_reset(P.tree_cnt + b * CSTRIDE);
  // validation; a bad parent is replaced by the root, so every chain ends
#pragma unroll
  for (int s = 0; s < WW_SLOTS; ++s) {
    const int i = s * WAVE + lane;
    st[s] = 0;
    if (i >= N) continue;
    if (yv[s] == -1) err |= SV_ERR_ROW;
    if (yv[s] == -2) err |= SV_ERR_INTERNAL;
    const bool bad = (i == 0) ? (pv[s] != -1) : (pv[s] < 0 || pv[s] >= i);
    if (bad) err |= SV_ERR_TREE;
    if (i > 0 && (cv[s] < 0 || cv[s] >= P.V)) err |= SV_ERR_TOKEN;
    pv[s] = bad ? 0 : pv[s];
    st[s] = bad ? 0 : 1;   // whether the match test applies
  }
  // The walk reads other nodes' parents, tokens, candidates and match flags by
  // index: from this wave's rows in LDS, one read each (a cross-lane permute per
  // slot instead made the walk take about 4 us).
  __shared__ int ww_sh[WPB][4][WAVE_WALK_NODES];
  int* sp = ww_sh[wave_in_block()][0];   // parents
  int* sc = ww_sh[wave_in_block()][1];   // candidates
  int* sy = ww_sh[wave_in_block()][2];   // tokens
  int* sm = ww_sh[wave_in_block()][3];   // match flags
#pragma unroll
  for (int s = 0; s < WW_SLOTS; ++s) {
    const int i = s * WAVE + lane;
    if (i < N) {
      sp[i] = pv[s];
      sc[i] = cv[s];
      sy[i] = yv[s];
    }
  }
  __builtin_amdgcn_wave_barrier();
  // match: the candidate is its parent's token (node indices are below N)
#pragma unroll
  for (int s = 0; s < WW_SLOTS; ++s) {
    const int i = s * WAVE + lane;
    const int yp = (i > 0 && i < N) ? sy[pv[s]] : 0;   // (the root has no parent to read)
    st[s] = (i > 0 && i < N && st[s] && cv[s] == yp) ? 1 : 0;
    if (i < N) sm[i] = st[s];
  }
  __builtin_amdgcn_wave_barrier();
  // every node's chain to the root: depth, and whether every node on it matched
  int cur[WW_SLOTS], d[WW_SLOTS], acc[WW_SLOTS];
  int too_deep = 0;
#pragma unroll
  for (int s = 0; s < WW_SLOTS; ++s) {
    const int i = s * WAVE + lane;
    cur[s] = i < N ? i : 0;
    d[s] = 0;
    acc[s] = i < N ? 1 : 0;
  }
  for (;;) {
    int moving = 0;
#pragma unroll
    for (int s = 0; s < WW_SLOTS; ++s) {
      const int m = sm[cur[s]];
      const int up = sp[cur[s]];
      if (cur[s] == 0) continue;
      if (d[s] >= P.max_depth) {
        too_deep = 1;
        cur[s] = 0;
        acc[s] = 0;
        continue;
      }
      acc[s] &= m;
      cur[s] = up;
      ++d[s];
      moving = 1;
    }
    if (__ballot(moving) == 0ull) break;
  }
  int best_key = -1;   // depth * 2^15 + (2^15 - 1 - index): deepest, then lowest index
#pragma unroll
  for (int s = 0; s < WW_SLOTS; ++s) {
    const int i = s * WAVE + lane;
    if (acc[s]) {
      const int key = (d[s] << 15) | (32767 - i);
      best_key = key > best_key ? key : best_key;
    }
  }
  best_key = wave_max_int(best_key);
  if (__ballot(too_deep) != 0ull) err |= SV_ERR_TREE;
  err = wave_or_int(err);
  int32_t* path = P.path_nodes + b * P.max_depth;
  int32_t* out = P.out_tokens + b * (P.max_depth + 1);
  if (err) {
    for (int64_t j = lane; j < P.max_depth; j += WAVE) path[j] = -1;
    for (int64_t j = lane; j <= P.max_depth; j += WAVE) out[j] = -1;
    if (lane == 0) {
      P.accept_len[b] = -1;
      if (P.err_flags) P.err_flags[b] = err;
    }
    return;
  }
  const int L = best_key >> 15;
  const int best = 32767 - (best_key & 32767);
  for (int64_t j = L + lane; j < P.max_depth; j += WAVE) path[j] = -1;
  for (int64_t j = L + 1 + lane; j <= P.max_depth; j += WAVE) out[j] = -1;
  // the accepted path, from the deepest node up
  int node = best;
  const int yb = sy[best];
  for (int j = L - 1; j >= 0; --j) {
    const int cn = sc[node];
    const int up = sp[node];
    if (lane == 0) {
      path[j] = node;
      out[j] = cn;
    }
    node = up;
  }
  if (lane == 0) {
    out[L] = yb;
    P.accept_len[b] = L;
    if (P.err_flags) P.err_flags[b] = 0;
  }
}

// Typical acceptance, gather wave g: lane l takes node t = 64 g + l of the batch
// and reads its candidate's logit in its parent's row (0 where the parent or the
// candidate is out of range: the walk flags those). Many waves across the chip
// keep these scattered reads in flight together; they run ahead of the stream.
template <int DT>
__device__ __forceinline__ void tree_gather_candidates(const TreeParams& P, int64_t g) {
  constexpr int E = DTraits<DT>::E;
  const int64_t t = g * WAVE + lane_id();
  if (t >= P.B * P.N) return;
  const int64_t b = t / P.N, i = t - b * P.N;
  float x = 0.0f;
  if (i > 0) {
    const int32_t pi = P.parent[b * P.parent_stride + i];
    const int32_t ci = P.cand[t];
    if (pi >= 0 && pi < i && ci >= 0 && ci < P.V) x = load_elem<DT>(P.logits + ((b * P.N + pi) * P.V) * E, ci);
  }
  P.xl[t] = x;
}

// ROWS: one wave per row (P.row_waves), a separate instantiation so that the
// chunk waves keep their own register budget.
template <int DT, int TD, bool ROWS>
__global__ __launch_bounds__(BLOCK) void tree_stream_kernel(TreeParams P) {
  constexpr int E = DTraits<DT>::E;
  constexpr bool STOCH = TD != TD_ARGMAX;
  int64_t w = (int64_t)blockIdx.x * WPB + wave_in_block();
  if constexpr (TD == TD_TYPICAL) {
    if (w < P.n_gather) {
      tree_gather_candidates<DT>(P, w);
      return;
    }
    w -= P.n_gather;
  }
  if (w >= P.n_stream) return;
  // row waves: wave w streams row w; chunk waves: see stream_coords
  int64_t q = w, c = 0;
  if constexpr (!ROWS) {
    uint32_t q32, c32;
    stream_coords((uint32_t)w, (uint32_t)P.CP, (uint32_t)(P.B * P.N), q32, c32);
    if (c32 >= (uint32_t)P.C) return;   // padding wave
    q = q32;
    c = c32;
  }
  const char* row = P.logits + (q * P.V) * E;
  if constexpr (TD == TD_TYPICAL) {
    EntParts ep;
    if (tree_typical_parts<DT, ROWS>(P, row, q, c, ep)) tree_typical_combine(P, q, ep);
    return;
  }
  RowParts rp;
  if constexpr (ROWS) {
    const int lane = lane_id();
#pragma unroll
    for (int t = 0; t < MAX_ROUNDS; ++t) {
      rp.m[t] = -INFINITY;
      rp.idx[t] = INT_SENTINEL;
      rp.s[t] = 0.0;
    }
    rp.got = true;
    rp.xin = false;
    rp.xv = 0.0f;
    row_chunks<DT>(row, P.V, P.C,
                   [&](const Chunk& k, const Raw& r) { return chunk_reduce<DT, STOCH, !STOCH>(k, r, P.c0, -1); },
                   [&](int cc, const Partial& p) {
#pragma unroll
                     for (int t = 0; t < MAX_ROUNDS; ++t)
                       if (t * WAVE + lane == cc) {
                         rp.m[t] = p.m;
                         rp.idx[t] = p.idx;
                         rp.s[t] = p.s;
                       }
                   });
  } else {
    const Partial p = chunk_partial<DT, STOCH, !STOCH>(row, P.V, c, P.c0);
    // Eager draws: the count before the record (a returning atomic also waits for
    // the stores issued before it; the reader polls the record's tag, so the order
    // is free), and the partials cleared after the draw, whose reload would wait
    // for those stores as well. The argmax measured faster the other way (C4
    // greedy 0.6 µs): it has no reload, and its clearing stores then complete
    // while the count's round trip runs.
    uint32_t old = 0;
    if (lane_id() == 0) {
      if constexpr (TD == TD_EAGER) {
        old = counter_add(P.row_cnt + q * CSTRIDE, 1u);
        put_rec(P.parts + (q * P.C + c) * PART_WORDS, p, P.tag);
      } else {
        put_rec(P.parts + (q * P.C + c) * PART_WORDS, p, P.tag);
        old = counter_add(P.row_cnt + q * CSTRIDE, 1u);
      }
    }
    old = bcast(old);
    if (old + 1 != (uint32_t)P.C) return;
    rp = read_parts(P.parts + q * P.C * PART_WORDS, P.C, P.tag);
    if constexpr (TD != TD_EAGER) clear_parts<Partial>(P.parts + q * P.C * PART_WORDS, P.C, P.row_cnt + q * CSTRIDE);
  }
  double wl[MAX_ROUNDS];
  const RowSums rs = row_sums<STOCH>(rp, P.c0, wl);
  // the node's token (TD_LAZY: 0 for a usable row); -1 an unusable row, -2 a
  // wait timed out
  int y;
  if (!rp.got) {
    y = -2;
  } else if constexpr (STOCH) {
    const bool usable = rs.M > -INFINITY && __builtin_isfinite(rs.Z) && rs.Z > 0.0;
    if constexpr (TD == TD_EAGER)
      y = usable ? softmax_draw<DT>(row, P.V, P.C, P.c0, P.uniforms[q], rp, rs, wl) : -1;
    else
      y = usable ? 0 : -1;
  } else {
    y = rs.argmax;
  }
  if constexpr (TD == TD_ARGMAX || TD == TD_EAGER) {
    if (P.wave_walk) {
      const int64_t b = q / P.N;
      uint32_t told = 0;
      if (lane_id() == 0) {
        told = counter_add(P.tree_cnt + b * CSTRIDE, 1u);
        Token t;
        t.y = y;
        put_rec(P.yrec + q, t, P.tag);
      }
      constexpr bool own = !ROWS && TD == TD_EAGER;   // this row's partials still to clear
      if (bcast(told) + 1 == (uint32_t)P.N) {
        tree_wave_walk(P, b, own ? q : -1);
        return;
      }
      if constexpr (own) clear_parts<Partial>(P.parts + q * P.C * PART_WORDS, P.C, P.row_cnt + q * CSTRIDE);
      return;
    }
  }
  if (lane_id() == 0) P.node_y[q] = y;
  if constexpr (!ROWS && TD == TD_EAGER) clear_parts<Partial>(P.parts + q * P.C * PART_WORDS, P.C, P.row_cnt + q * CSTRIDE);
}

// node indices and depths fit the 15-bit fields of the walk's search keys
static_assert(SV_MAX_TREE_NODES <= 16384, "tree walk keys");
constexpr int WALK_BATCH = 8;   // nodes per thread whose loads are in flight together

// OR over the workgroup (sh: one int per wave).
template <int NT>
__device__ __forceinline__ int block_or(int v, int* sh) {
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) v |= __shfl_xor(v, o);
  if (lane_id() == 0) sh[wave_in_block()] = v;
  __syncthreads();
  int r = 0;
  for (int wv = 0; wv < NT / WAVE; ++wv) r |= sh[wv];
  __syncthreads();
  return r;
}

// Largest v over the workgroup (sh: one int per wave).
template <int NT>
__device__ __forceinline__ int block_max_int(int v, int* sh) {
  v = wave_max_int(v);
  if (lane_id() == 0) sh[wave_in_block()] = v;
  __syncthreads();
  int r = sh[0];
  for (int wv = 1; wv < NT / WAVE; ++wv) r = sh[wv] > r ? sh[wv] : r;
  __syncthreads();
  return r;
}

// Inverse-CDF draw from softmax(row / T) with uniform u by the whole workgroup:
// the waves reduce the chunks (the same partials the streaming pass forms), then
// wave 0 picks the chunk and scans it. The token is valid in wave 0.
template <int DT, int NT>
__device__ __forceinline__ int walk_draw(const char* row, int64_t V, int C, float c0, float u,
                                         float* pm, double* ps) {
  const int wv = wave_in_block(), lane = lane_id();
  for (int c = wv; c < C; c += NT / WAVE) {
    const Partial p = chunk_partial<DT, true, false>(row, V, c, c0);
    if (lane == 0) {
      pm[c] = p.m;
      ps[c] = p.s;
    }
  }
  __syncthreads();
  int y = -1;
  if (wv == 0) {
    RowParts rp;
#pragma unroll
    for (int t = 0; t < MAX_ROUNDS; ++t) {
      const int c = t * WAVE + lane;
      rp.m[t] = c < C ? pm[c] : -INFINITY;
      rp.idx[t] = INT_SENTINEL;
      rp.s[t] = c < C ? ps[c] : 0.0;
    }
    rp.got = true;
    rp.xin = false;
    rp.xv = 0.0f;
    double wl[MAX_ROUNDS];
    const RowSums rs = row_sums<true>(rp, c0, wl);
    if (rs.Z > 0.0 && __builtin_isfinite(rs.Z)) y = softmax_draw<DT>(row, V, C, c0, u, rp, rs, wl);
  }
  __syncthreads();   // the partial arrays are reused by the next draw
  return y;
}

// Walk modes: the node tokens are known (greedy, or drawn while streaming); LAZY
// draws the tokens of the accepted nodes level by level; TYPICAL accepts a node
// when its candidate's probability under its parent's distribution clears the
// parent's threshold, and draws only the final token.
enum WalkMode { WM_KNOWN = 0, WM_LAZY = 1, WM_TYPICAL = 2 };

// Accepted-path search of tree b (one workgroup of NT threads). LDS: parent
// (int16) and one state byte per node. WM_KNOWN / WM_TYPICAL: a node is accepted
// when every node on its path matches (its token equals its parent's, or its
// candidate passes the parent's threshold); the deepest such node, lowest index on
// ties, ends the path. WM_LAZY: the walk goes level by level from the root, drawing
// the token of each accepted node and accepting the children whose candidate
// equals it.
template <int DT, int WM, int NT>
__global__ __launch_bounds__(NT) void tree_walk_kernel(TreeParams args) {
  (void)args;
  const TreeParams& P = kernel_args<TreeParams>();
  constexpr int E = DTraits<DT>::E;
  constexpr bool DRAWS = WM != WM_KNOWN;
  extern __shared__ unsigned char smem[];
  __shared__ int red_sh[NT / WAVE];
  __shared__ float pm_sh[DRAWS ? MAX_CHUNKS : 1];
  __shared__ double ps_sh[DRAWS ? MAX_CHUNKS : 1];
  const int64_t b = blockIdx.x;
  const int64_t N = P.N;
  int16_t* par_s = reinterpret_cast<int16_t*>(smem);
  unsigned char* st_s = smem + 2 * N;   // match flag; WM_LAZY: 0 / 1 accepted / 2 drawn
  const int32_t* par = P.parent + b * P.parent_stride;
  const int32_t* cand = P.cand + b * N;
  int32_t* ny = P.node_y + b * N;
  const int tid = threadIdx.x;
  int err = 0;
  // validation (and the match flags), WALK_BATCH nodes per thread at a time
  for (int64_t base = 0; base < N; base += (int64_t)NT * WALK_BATCH) {
    int yv[WALK_BATCH], pv[WALK_BATCH], cv[WALK_BATCH], yp[WALK_BATCH];
    float xl[WALK_BATCH], nm[WALK_BATCH];
    double ng[WALK_BATCH];
    int nok[WALK_BATCH];
#pragma unroll
    for (int j = 0; j < WALK_BATCH; ++j) {
      const int64_t i = base + (int64_t)j * NT + tid;
      yv[j] = 0;
      pv[j] = -1;
      cv[j] = 0;
      if (i < N) {
        yv[j] = ny[i];
        pv[j] = par[i];
        cv[j] = cand[i];
      }
    }
#pragma unroll
    for (int j = 0; j < WALK_BATCH; ++j) {
      const int64_t i = base + (int64_t)j * NT + tid;
      const bool ok = i > 0 && i < N && pv[j] >= 0 && pv[j] < i;
      yp[j] = -1;
      xl[j] = nm[j] = 0.0f;
      ng[j] = 0.0;
      nok[j] = 0;
      if (WM == WM_KNOWN && ok) yp[j] = ny[pv[j]];
      if (WM == WM_TYPICAL && ok && cv[j] >= 0 && cv[j] < P.V) {
        // the candidate's logit in its parent's row, and the parent's statistics
        const NodeStat ps = P.nstat[b * N + pv[j]];
        ng[j] = ps.G;
        nm[j] = ps.M;
        nok[j] = ps.ok;
        xl[j] = P.xl[b * N + i];
      }
    }
#pragma unroll
    for (int j = 0; j < WALK_BATCH; ++j) {
      const int64_t i = base + (int64_t)j * NT + tid;
      if (i >= N) continue;
      if (yv[j] == -1) err |= SV_ERR_ROW;
      if (yv[j] == -2) err |= SV_ERR_INTERNAL;
      const bool bad = (i == 0) ? (pv[j] != -1) : (pv[j] < 0 || pv[j] >= i);
      par_s[i] = (int16_t)(bad ? 0 : pv[j]);
      if (bad) err |= SV_ERR_TREE;
      unsigned char m = 0;
      if (i > 0) {
        if (cv[j] < 0 || cv[j] >= P.V) err |= SV_ERR_TOKEN;
        if (WM == WM_KNOWN && !bad) m = (cv[j] == yp[j]) ? 1 : 0;
        if (WM == WM_TYPICAL && !bad && nok[j]) {
          // p_parent(cand) against the parent's threshold, through its gate
          m = ((double)xl[j] - (double)nm[j]) * (double)P.c0 > ng[j] ? 1 : 0;
        }
      }
      st_s[i] = WM == WM_LAZY ? (unsigned char)(i == 0 ? 1 : 0) : m;
    }
  }
  int all_err = block_or<NT>(err, red_sh);
  // depth check (bad parents were replaced by the root, so every chain ends; the
  // bound is checked whatever other error was found) and, tokens known, the path
  // search; WALK_BATCH chains per thread advance together
  int best_key = -1;   // depth * 2^15 + (2^15 - 1 - index): deepest, then lowest index
  int too_deep = 0;
  for (int64_t base = 0; base < N; base += (int64_t)NT * WALK_BATCH) {
    int cur[WALK_BATCH], d[WALK_BATCH], acc[WALK_BATCH];
#pragma unroll
    for (int j = 0; j < WALK_BATCH; ++j) {
      const int64_t i = base + (int64_t)j * NT + tid;
      cur[j] = i < N ? (int)i : 0;
      d[j] = 0;
      acc[j] = i < N ? 1 : 0;
    }
    for (;;) {
      int moving = 0;
#pragma unroll
      for (int j = 0; j < WALK_BATCH; ++j) {
        if (cur[j] == 0) continue;
        if (d[j] >= P.max_depth) {
          too_deep = 1;
          cur[j] = 0;
          acc[j] = 0;
          continue;
        }
        if (WM != WM_LAZY) acc[j] &= st_s[cur[j]];
        cur[j] = par_s[cur[j]];
        ++d[j];
        moving = 1;
      }
      if (!moving) break;
    }
    if (WM != WM_LAZY) {
#pragma unroll
      for (int j = 0; j < WALK_BATCH; ++j) {
        const int64_t i = base + (int64_t)j * NT + tid;
        if (acc[j]) {
          const int key = (d[j] << 15) | (int)(32767 - i);
          best_key = key > best_key ? key : best_key;
        }
      }
    }
  }
  if (__syncthreads_or(too_deep)) all_err |= SV_ERR_TREE;
  int32_t* path = P.path_nodes + b * P.max_depth;
  int32_t* out = P.out_tokens + b * (P.max_depth + 1);
  if (all_err) {
    for (int64_t j = tid; j < P.max_depth; j += NT) path[j] = -1;
    for (int64_t j = tid; j <= P.max_depth; j += NT) out[j] = -1;
    if (tid == 0) {
      P.accept_len[b] = -1;
      if (P.err_flags) P.err_flags[b] = all_err;
    }
  } else {
    int L = 0, best = 0;
    if constexpr (WM == WM_LAZY) {
      for (int level = 0;; ++level) {
        // draw the accepted nodes of this level, lowest index first
        int first = -1;
        for (;;) {
          int key = -1;   // 2^15 - 1 - index of an accepted node still to draw
          for (int64_t i = tid; i < N; i += NT)
            if (st_s[i] == 1) key = (int)(32767 - i) > key ? (int)(32767 - i) : key;
          key = block_max_int<NT>(key, red_sh);
          if (key < 0) break;
          const int f = 32767 - key;
          if (first < 0) first = f;
          const char* row = P.logits + ((b * N + f) * P.V) * E;
          const int y = walk_draw<DT, NT>(row, P.V, P.C, P.c0, P.uniforms[b * N + f], pm_sh, ps_sh);
          if (tid == 0) {
            ny[f] = y;
            st_s[f] = 2;
          }
          __syncthreads();
        }
        L = level;
        best = first;
        // accept the children whose candidate is their parent's drawn token
        int any = 0;
        for (int64_t i = 1 + tid; i < N; i += NT) {
          const int pi = par_s[i];
          // the drawn token was stored by thread 0 after this thread's first read of ny
          if (st_s[i] == 0 && st_s[pi] == 2 &&
              cand[i] == __hip_atomic_load(ny + pi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
            st_s[i] = 1;
            any = 1;
          }
        }
        if (!__syncthreads_or(any)) break;
      }
    } else {
      const int r = block_max_int<NT>(best_key, red_sh);
      L = r >> 15;
      best = 32767 - (r & 32767);
      if constexpr (WM == WM_TYPICAL) {
        // the final token: a draw from the last node's distribution
        const char* row = P.logits + ((b * N + best) * P.V) * E;
        const int y = walk_draw<DT, NT>(row, P.V, P.C, P.c0, P.uniforms[b * N + best], pm_sh, ps_sh);
        if (tid == 0) ny[best] = y;
        __syncthreads();
      }
    }
    for (int64_t j = L + tid; j < P.max_depth; j += NT) path[j] = -1;
    for (int64_t j = L + 1 + tid; j <= P.max_depth; j += NT) out[j] = -1;
    if (tid == 0) {
      int node = best;
      for (int j = L - 1; j >= 0; --j) {
        path[j] = node;
        out[j] = cand[node];
        node = par_s[node];
      }
      out[L] = ny[best];
      P.accept_len[b] = L;
      if (P.err_flags) P.err_flags[b] = 0;
    }
  }
  // leave the node tokens (and statistics) zero, as the workspace was
  __syncthreads();
  for (int64_t i = tid; i < N; i += NT) {
    ny[i] = 0;
    if (WM == WM_TYPICAL) {
      P.xl[b * N + i] = 0.0f;
      NodeStat z;
      z.G = 0.0;
      z.M = 0.0f;
      z.ok = 0;
      P.nstat[b * N + i] = z;
    }
  }
}

// ------------------------------------------------------------------ row statistics
struct RowStatsParams {
  const char* x;
  float* row_max;
  float* row_lse;
  int32_t* row_argmax;
  int32_t* err_flags;
  uint64_t* parts;
  uint32_t* row_cnt;
  int64_t rows, V;
  int C, CP;
  float c0;
  uint32_t tag;
  int64_t n_stream;
};

template <int DT>
__global__ __launch_bounds__(BLOCK) void row_stats_kernel(RowStatsParams P) {
  constexpr int E = DTraits<DT>::E;
  const int64_t w = (int64_t)blockIdx.x * WPB + wave_in_block();
  if (w >= P.n_stream) return;
  const uint32_t C = (uint32_t)P.C;
  uint32_t r32, c32;
  stream_coords((uint32_t)w, (uint32_t)P.CP, (uint32_t)P.rows, r32, c32);
  if (c32 >= C) return;   // padding wave
  const int64_t r = r32, c = c32;
  const char* row = P.x + (r * P.V) * E;
  const Partial p = chunk_partial<DT, true, true>(row, P.V, c, P.c0);
  // the count before the record: a returning atomic also waits for the stores
  // issued before it (the reader polls the record's tag, so the order is free)
  uint32_t old = 0;
  if (lane_id() == 0) {
    old = counter_add(P.row_cnt + r * CSTRIDE, 1u);
    put_rec(P.parts + (r * P.C + c) * PART_WORDS, p, P.tag);
  }
  old = bcast(old);
  if (old + 1 != C) return;
  const RowParts rp = read_parts(P.parts + r * P.C * PART_WORDS, P.C, P.tag);
  double wl[MAX_ROUNDS];
  const RowSums rs = row_sums<true>(rp, P.c0, wl);
  if (lane_id() == 0) {
    const bool ok = rp.got && rs.argmax >= 0 && __builtin_isfinite(rs.Z) && rs.Z > 0.0;
    if (P.row_max) P.row_max[r] = rs.M;
    if (P.row_argmax) P.row_argmax[r] = rs.argmax;
    if (P.row_lse) P.row_lse[r] = ok ? (float)((double)rs.M * (double)P.c0 * LN2 + log(rs.Z)) : NAN;
    if (P.err_flags) P.err_flags[r] = ok ? 0 : (!rp.got ? SV_ERR_INTERNAL : SV_ERR_ROW);
  }
  clear_parts<Partial>(P.parts + r * P.C * PART_WORDS, P.C, P.row_cnt + r * CSTRIDE);
}

__global__ __launch_bounds__(BLOCK) void clear_kernel(unsigned char* p, size_t bytes) {
  const size_t n16 = bytes / 16;
  const size_t stride = (size_t)gridDim.x * BLOCK;
  uint4* q = reinterpret_cast<uint4*>(p);
  for (size_t i = (size_t)blockIdx.x * BLOCK + threadIdx.x; i < n16; i += stride) q[i] = make_uint4(0, 0, 0, 0);
  for (size_t i = n16 * 16 + (size_t)blockIdx.x * BLOCK + threadIdx.x; i < bytes; i += stride) p[i] = 0;
}

// A plain streaming read of one or two buffers with nothing else done, to measure
// what reading the bytes of a verification costs by itself: one wave per 8 KiB
// chunk (its eight 16-byte loads per lane issued together, as in the streaming
// waves above), the chunk's largest 32-bit word stored to sink[wave]. Chunks
// [0, ca) are buffer a's, the rest buffer b's; na, nb count 16-byte units.
__global__ __launch_bounds__(BLOCK) void read_probe_kernel(const uint4* a, int64_t na, int64_t ca, const uint4* b,
                                                           int64_t nb, int64_t nwaves, uint32_t* sink) {
  const int64_t w = (int64_t)blockIdx.x * WPB + wave_in_block();
  if (w >= nwaves) return;
  const int lane = lane_id();
  const bool in_a = w < ca;
  const uint4* p = in_a ? a : b;
  const int64_t n = in_a ? na : nb;
  const int64_t u0 = (in_a ? w : w - ca) * CHUNK_UNITS;
  uint4 v[CU];
  if (u0 + CHUNK_UNITS <= n) {
#pragma unroll
    for (int j = 0; j < CU; ++j) v[j] = p[u0 + j * WAVE + lane];
  } else {
#pragma unroll
    for (int j = 0; j < CU; ++j) {
      const int64_t u = u0 + j * WAVE + lane;
      v[j] = u < n ? p[u] : make_uint4(0, 0, 0, 0);
    }
  }
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < CU; ++j) m = max(m, max(max(v[j].x, v[j].y), max(v[j].z, v[j].w)));
#pragma unroll
  for (int o = WAVE / 2; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  if (lane == 0) sink[w] = m;
}

// ------------------------------------------------------------------ host side
struct LinearShape {
  int64_t R, RQ, C, RW;
};

inline LinearShape linear_shape(int64_t B, int64_t k, int64_t V, sv_dtype dt, sv_mode mode) {
  LinearShape s;
  const bool stoch = mode == SV_STOCHASTIC;
  s.R = stoch ? 2 * k + 1 : k + 1;
  s.RQ = B * s.R;
  s.C = chunks_per_row(V, dt);
  s.RW = stoch ? 4 : 2;
  return s;
}

Layout linear_layout(int64_t B, int64_t k, int64_t V, sv_dtype dt, sv_mode mode) {
  const LinearShape s = linear_shape(B, k, V, dt, mode);
  const size_t RG = mode == SV_STOCHASTIC ? (size_t)(B * s.C * RH) : 0;   // residual waves (stochastic only)
  return make_layout({(size_t)(s.RQ * s.C * s.RW) * 8, (size_t)(B * k) * PST_WORDS * 8, (size_t)B * ROW_WORDS * 8,
                      RG * DEC_WORDS * 8, RG * RES_WORDS * 8, (size_t)B * 8,
                      (size_t)(B * SSTRIDE) * 8, (size_t)(B * CSTRIDE) * 4,
                      (size_t)(B * CSTRIDE) * 4, (size_t)(B * CSTRIDE) * 4, (size_t)(B * k) * PROB_WORDS * 8,
                      RG * VERD_WORDS * 8, (size_t)8});
}

Layout tree_layout(int64_t B, int64_t N, int64_t V, sv_dtype dt) {
  const int64_t C = chunks_per_row(V, dt);
  return make_layout({(size_t)(B * N * C) * PART_WORDS * 8, (size_t)(B * N * CSTRIDE) * 4, (size_t)(B * N) * 4,
                      (size_t)(B * N) * sizeof(NodeStat), (size_t)(B * N) * 8, (size_t)(B * CSTRIDE) * 4,
                      (size_t)(B * N) * 4});
}

Layout rowstats_layout(int64_t rows, int64_t V, sv_dtype dt) {
  const int64_t C = chunks_per_row(V, dt);
  return make_layout({(size_t)(rows * C) * PART_WORDS * 8, (size_t)(rows * CSTRIDE) * 4});
}

template <int DT, bool STOCH>
struct LinearLauncher {
  static sv_status run(const LinearParams& P, hipStream_t s) {
    hipLaunchKernelGGL((linear_kernel<DT, STOCH>), dim3(blocks_for(P.n_waves)), dim3(BLOCK), 0, s, P);
    return launch_status();
  }
};

// Walk workgroups: 1024 threads, so that one pass of WALK_BATCH nodes per thread
// covers trees of up to 8192 nodes.
template <int DT, bool STOCH>
struct TreeLauncher {
  static sv_status run(const TreeParams& P, size_t smem, hipStream_t s) {
    const bool eager = STOCH && P.B * P.N <= TREE_EAGER_ROWS;
    const dim3 grid(blocks_for(P.n_stream)), trees((unsigned)P.B);
    TreeParams Q = P;
    Q.wave_walk = (!STOCH || eager) && P.N <= WAVE_WALK_NODES;
    if (!STOCH) {
      if (P.row_waves)
        hipLaunchKernelGGL((tree_stream_kernel<DT, TD_ARGMAX, true>), grid, dim3(BLOCK), 0, s, Q);
      else
        hipLaunchKernelGGL((tree_stream_kernel<DT, TD_ARGMAX, false>), grid, dim3(BLOCK), 0, s, Q);
    } else if (eager) {
      hipLaunchKernelGGL((tree_stream_kernel<DT, TD_EAGER, false>), grid, dim3(BLOCK), 0, s, Q);
    } else {
      if (P.row_waves)
        hipLaunchKernelGGL((tree_stream_kernel<DT, TD_LAZY, true>), grid, dim3(BLOCK), 0, s, Q);
      else
        hipLaunchKernelGGL((tree_stream_kernel<DT, TD_LAZY, false>), grid, dim3(BLOCK), 0, s, Q);
    }
    if (launch_status() != SV_OK) return SV_EHIP;
    if (Q.wave_walk) return SV_OK;   // the streaming launch has walked every tree
    if (STOCH && !eager) {
      hipLaunchKernelGGL((tree_walk_kernel<DT, WM_LAZY, 1024>), trees, dim3(1024), smem, s, P);
    } else {
      hipLaunchKernelGGL((tree_walk_kernel<DT, WM_KNOWN, 1024>), trees, dim3(1024), smem, s, P);
    }
    return launch_status();
  }
};

template <int DT, bool UNUSED>
struct TypicalLauncher {
  static sv_status run(const TreeParams& P, size_t smem, hipStream_t s) {
    // gather waves ahead of the streaming waves, whole groups of 8 workgroups so
    // that the streaming waves keep their XCD placement
    TreeParams Q = P;
    Q.n_gather = ((P.B * P.N + WAVE - 1) / WAVE + 8 * WPB - 1) / (8 * WPB) * (8 * WPB);
    if (P.row_waves)
      hipLaunchKernelGGL((tree_stream_kernel<DT, TD_TYPICAL, true>), dim3(blocks_for(Q.n_gather + P.n_stream)),
                         dim3(BLOCK), 0, s, Q);
    else
      hipLaunchKernelGGL((tree_stream_kernel<DT, TD_TYPICAL, false>), dim3(blocks_for(Q.n_gather + P.n_stream)),
                         dim3(BLOCK), 0, s, Q);
    if (launch_status() != SV_OK) return SV_EHIP;
    hipLaunchKernelGGL((tree_walk_kernel<DT, WM_TYPICAL, 1024>), dim3((unsigned)P.B), dim3(1024), smem, s, Q);
    return launch_status();
  }
};

template <int DT, bool UNUSED>
struct RowStatsLauncher {
  static sv_status run(const RowStatsParams& P, hipStream_t s) {
    hipLaunchKernelGGL((row_stats_kernel<DT>), dim3(blocks_for(P.n_stream)), dim3(BLOCK), 0, s, P);
    return launch_status();
  }
};

// Waves of the stochastic linear kernel for dtype `dt` that can be resident on
// the current device at once (0 if the runtime cannot tell), cached per device.
constexpr int CAP_DEVICES = 64;
static std::atomic<int64_t> g_capacity[CAP_DEVICES][3];

inline int64_t stochastic_wave_capacity(sv_dtype dt) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= CAP_DEVICES || !dtype_ok(dt)) return 0;
  const int64_t c = g_capacity[dev][dt].load(std::memory_order_relaxed);
  if (c > 0) return c;
  const void* fn = dt == SV_F32 ? reinterpret_cast<const void*>(&linear_kernel<DT_F32, true>)
                 : dt == SV_BF16 ? reinterpret_cast<const void*>(&linear_kernel<DT_BF16, true>)
                                 : reinterpret_cast<const void*>(&linear_kernel<DT_F16, true>);
  int blocks = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, BLOCK, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  const int64_t cap = (int64_t)blocks * cus * WPB;
  g_capacity[dev][dt].store(cap, std::memory_order_relaxed);
  return cap;
}

// Checks and fills the parameters of the linear entry points (B == 0: SV_OK with
// nothing to launch).
sv_status linear_setup(LinearParams& P, sv_mode mode, float temperature, int64_t B, int64_t k, int64_t V,
                       sv_dtype dtype, const void* target_logits, const void* draft_logits,
                       const int32_t* draft_tokens, const float* uniforms, int32_t* accept_len,
                       int32_t* out_tokens, float* p_target, float* p_draft, int32_t* err_flags,
                       void* workspace, size_t workspace_bytes) {
  if (!dtype_ok(dtype)) return SV_EDTYPE;
  if (mode != SV_GREEDY && mode != SV_STOCHASTIC) return SV_EINVAL;
  const bool stoch = (mode == SV_STOCHASTIC);
  if (B < 0 || k < 0 || V < 1) return SV_EINVAL;
  if (k > SV_MAX_K || !shape_ok(V, dtype)) return SV_ELIMIT;
  if (B == 0) return SV_OK;
  if (!target_logits || !accept_len || !out_tokens || (k > 0 && !draft_tokens)) return SV_EINVAL;
  if (stoch && (!temperature_ok(temperature) || !uniforms || (k > 0 && !draft_logits))) return SV_EINVAL;
  const Layout lay = linear_layout(B, k, V, dtype, mode);
  if (!ws_ok(workspace, workspace_bytes, lay.total)) return SV_EWORKSPACE;
  P.target = static_cast<const char*>(target_logits);
  P.draft = static_cast<const char*>(draft_logits);
  P.tokens = draft_tokens;
  P.uniforms = uniforms;
  P.accept_len = accept_len;
  P.out_tokens = out_tokens;
  P.p_target = stoch ? p_target : nullptr;
  P.p_draft = stoch ? p_draft : nullptr;
  P.err_flags = err_flags;
  const LinearShape sh = linear_shape(B, k, V, dtype, mode);
  char* ws = static_cast<char*>(workspace);
  P.seg = reinterpret_cast<uint64_t*>(ws + lay.off[0]);
  P.pst = reinterpret_cast<uint64_t*>(ws + lay.off[1]);
  P.rks = reinterpret_cast<uint64_t*>(ws + lay.off[2]);
  P.dec = reinterpret_cast<uint64_t*>(ws + lay.off[3]);
  P.res = reinterpret_cast<uint64_t*>(ws + lay.off[4]);
  P.tok = reinterpret_cast<uint64_t*>(ws + lay.off[5]);
  P.state = reinterpret_cast<uint64_t*>(ws + lay.off[6]);
  P.fin = reinterpret_cast<uint32_t*>(ws + lay.off[7]);
  P.res_cnt = reinterpret_cast<uint32_t*>(ws + lay.off[8]);
  P.slots = reinterpret_cast<uint64_t*>(ws + lay.off[12]);
  P.errw = reinterpret_cast<uint32_t*>(ws + lay.off[9]);
  P.prob = reinterpret_cast<uint64_t*>(ws + lay.off[10]);
  P.verd = reinterpret_cast<uint64_t*>(ws + lay.off[11]);
  P.B = B;
  P.k = k;
  P.V = V;
  P.C = (int)sh.C;
  P.RW = (int)sh.RW;
  P.EV = (int)(k + 2);
  P.c0 = stoch ? temperature_c0(temperature) : 1.0f;
  // residual waves: RH per chunk (they come after the position blocks); hold mode
  // when all of them fit on the GPU at once, with room to spare, else queued
  P.CG = RH * P.C;
  P.hold = stoch && k > 0 && B * P.CG <= stochastic_wave_capacity(dtype) / 2;
  P.queue = stoch && k > 0 && !P.hold;
  // Residual waves dispatched before target row k streams, so that the reloads and
  // draws of the sequences rejected first overlap that stream instead of following
  // it: in hold mode every sequence's, in a queued launch those of the first
  // decision slots (the first sequences rejected), at most a quarter of the
  // resident waves. They wait only for pair decisions, made by waves dispatched
  // before them.
  P.early = P.hold ? (uint32_t)B : 0u;
  if (P.queue) {
    const int64_t cap = stochastic_wave_capacity(dtype) / 4 / P.CG;
    P.early = (uint32_t)std::max<int64_t>(0, std::min<int64_t>({B, (int64_t)EARLY_SLOTS, cap}));
  }
  // see linear_role for the order of the waves
  if (!stoch) {
    P.n_waves = sh.RQ * sh.C + B;
    P.tk0 = 0;
  } else {
    const int64_t CG = k > 0 ? P.CG : 0;
    P.tk0 = (uint32_t)(k * B * (2 * sh.C + 1));
    P.n_waves = P.tk0 + B * (sh.C + 1 + CG);
  }
  if (P.n_waves > MAX_WAVES) return SV_ELIMIT;
  P.commit = false;
  P.tag = next_tag();
  return SV_OK;
}

// Checks and fills the parameters shared by the tree entry points (B == 0: SV_OK
// with nothing to launch).
sv_status tree_setup(TreeParams& P, size_t& smem, bool stoch, float temperature, int64_t B, int64_t n_nodes,
                     int64_t V, sv_dtype dtype, const int32_t* parent, int64_t parent_batch_stride,
                     const int32_t* cand_tokens, const void* target_logits, const float* uniforms,
                     int64_t max_depth, int32_t* accept_len, int32_t* path_nodes, int32_t* out_tokens,
                     int32_t* err_flags, void* workspace, size_t workspace_bytes) {
  if (B < 0 || n_nodes < 1 || V < 1 || max_depth < 0 || parent_batch_stride < 0) return SV_EINVAL;
  if (n_nodes > SV_MAX_TREE_NODES || !shape_ok(V, dtype)) return SV_ELIMIT;
  if (B == 0) return SV_OK;
  if (!parent || !cand_tokens || !target_logits || !accept_len || !out_tokens) return SV_EINVAL;
  if (max_depth > 0 && !path_nodes) return SV_EINVAL;
  if (stoch && (!temperature_ok(temperature) || !uniforms)) return SV_EINVAL;
  const Layout lay = tree_layout(B, n_nodes, V, dtype);
  if (!ws_ok(workspace, workspace_bytes, lay.total)) return SV_EWORKSPACE;
  P.logits = static_cast<const char*>(target_logits);
  P.parent = parent;
  P.parent_stride = parent_batch_stride;
  P.cand = cand_tokens;
  P.uniforms = uniforms;
  P.accept_len = accept_len;
  P.path_nodes = path_nodes;
  P.out_tokens = out_tokens;
  P.err_flags = err_flags;
  char* ws = static_cast<char*>(workspace);
  P.parts = reinterpret_cast<uint64_t*>(ws + lay.off[0]);
  P.row_cnt = reinterpret_cast<uint32_t*>(ws + lay.off[1]);
  P.node_y = reinterpret_cast<int32_t*>(ws + lay.off[2]);
  P.nstat = reinterpret_cast<NodeStat*>(ws + lay.off[3]);
  P.yrec = reinterpret_cast<uint64_t*>(ws + lay.off[4]);
  P.tree_cnt = reinterpret_cast<uint32_t*>(ws + lay.off[5]);
  P.xl = reinterpret_cast<float*>(ws + lay.off[6]);
  P.wave_walk = false;
  P.n_gather = 0;
  P.B = B;
  P.N = n_nodes;
  P.V = V;
  P.max_depth = max_depth;
  P.C = (int)chunks_per_row(V, dtype);
  P.CP = (P.C + WPB - 1) / WPB * WPB;
  P.c0 = stoch ? temperature_c0(temperature) : 1.0f;
  // more rows than one launch of chunk waves fills the chip with: one wave per row
  P.row_waves = B * n_nodes > TREE_EAGER_ROWS;
  P.n_stream = P.row_waves ? B * n_nodes : B * n_nodes * P.CP;
  if (B * n_nodes * P.CP > MAX_WAVES || B > 0x7fffffffLL) return SV_ELIMIT;
  P.tag = next_tag();
  // LDS of the path search: parent (2 B) + match flag (1 B) per node
  smem = (size_t)((3 * n_nodes + 15) & ~(int64_t)15);
  return SV_OK;
}

}  // namespace

extern "C" {

const char* spec_verify_status_string(sv_status s) {
  switch (s) {
    case SV_OK: return "ok";
    case SV_EINVAL: return "invalid argument";
    case SV_EDTYPE: return "unknown dtype";
    case SV_EWORKSPACE: return "workspace missing, misaligned or too small";
    case SV_EHIP: return "HIP launch failed";
    case SV_ELIMIT: return "shape beyond a documented limit";
  }
  return "unknown status";
}

size_t spec_verify_linear_workspace(int64_t B, int64_t k, int64_t V, sv_dtype dtype, sv_mode mode) {
  if (B < 0 || k < 0 || V < 1 || !dtype_ok(dtype)) return 0;
  return linear_layout(B, k, V, dtype, mode).total;
}

sv_status spec_verify_linear(sv_mode mode, float temperature, int64_t B, int64_t k, int64_t V,
                             sv_dtype dtype, const void* target_logits, const void* draft_logits,
                             const int32_t* draft_tokens, const float* uniforms, int32_t* accept_len,
                             int32_t* out_tokens, float* p_target, float* p_draft,
                             int32_t* err_flags, void* workspace, size_t workspace_bytes,
                             sv_stream_t stream) {
  LinearParams P{};
  const sv_status st = linear_setup(P, mode, temperature, B, k, V, dtype, target_logits, draft_logits, draft_tokens,
                                    uniforms, accept_len, out_tokens, p_target, p_draft, err_flags, workspace,
                                    workspace_bytes);
  if (st != SV_OK || B == 0) return st;
  return dispatch<LinearLauncher>(dtype, mode == SV_STOCHASTIC, P, reinterpret_cast<hipStream_t>(stream));
}

sv_status spec_verify_linear_commit(sv_mode mode, float temperature, int64_t B, int64_t k, int64_t V,
                                    sv_dtype dtype, const void* target_logits, const void* draft_logits,
                                    const int32_t* draft_tokens, const float* uniforms, int32_t* accept_len,
                                    int32_t* out_tokens, float* p_target, float* p_draft, int32_t* err_flags,
                                    int32_t* seq_len, int32_t* history, int64_t capacity, int32_t* shifted,
                                    int32_t* next_token, void* workspace, size_t workspace_bytes,
                                    sv_stream_t stream) {
  if (capacity < 0) return SV_EINVAL;
  LinearParams P{};
  const sv_status st = linear_setup(P, mode, temperature, B, k, V, dtype, target_logits, draft_logits, draft_tokens,
                                    uniforms, accept_len, out_tokens, p_target, p_draft, err_flags, workspace,
                                    workspace_bytes);
  if (st != SV_OK || B == 0) return st;
  if (!seq_len || (capacity > 0 && !history)) return SV_EINVAL;
  P.commit = true;
  P.seq_len = seq_len;
  P.history = capacity > 0 ? history : nullptr;
  P.capacity = capacity;
  P.shifted = shifted;
  P.next_token = next_token;
  return dispatch<LinearLauncher>(dtype, mode == SV_STOCHASTIC, P, reinterpret_cast<hipStream_t>(stream));
}

size_t spec_verify_tree_workspace(int64_t B, int64_t n_nodes, int64_t V, sv_dtype dtype, sv_mode mode) {
  (void)mode;
  if (B < 0 || n_nodes < 1 || V < 1 || !dtype_ok(dtype)) return 0;
  return tree_layout(B, n_nodes, V, dtype).total;
}

sv_status spec_verify_tree(sv_mode mode, float temperature, int64_t B, int64_t n_nodes, int64_t V,
                           sv_dtype dtype, const int32_t* parent, int64_t parent_batch_stride,
                           const int32_t* cand_tokens, const void* target_logits,
                           const float* uniforms, int64_t max_depth, int32_t* accept_len,
                           int32_t* path_nodes, int32_t* out_tokens, int32_t* err_flags,
                           void* workspace, size_t workspace_bytes, sv_stream_t stream) {
  if (!dtype_ok(dtype)) return SV_EDTYPE;
  if (mode != SV_GREEDY && mode != SV_STOCHASTIC) return SV_EINVAL;
  const bool stoch = (mode == SV_STOCHASTIC);
  TreeParams P{};
  size_t smem = 0;
  const sv_status st = tree_setup(P, smem, stoch, temperature, B, n_nodes, V, dtype, parent, parent_batch_stride,
                                  cand_tokens, target_logits, uniforms, max_depth, accept_len, path_nodes,
                                  out_tokens, err_flags, workspace, workspace_bytes);
  if (st != SV_OK || B == 0) return st;
  return dispatch<TreeLauncher>(dtype, stoch, P, smem, reinterpret_cast<hipStream_t>(stream));
}

sv_status spec_verify_tree_typical(float temperature, double epsilon, double delta, int64_t B, int64_t n_nodes,
                                   int64_t V, sv_dtype dtype, const int32_t* parent,
                                   int64_t parent_batch_stride, const int32_t* cand_tokens,
                                   const void* target_logits, const float* uniforms, int64_t max_depth,
                                   int32_t* accept_len, int32_t* path_nodes, int32_t* out_tokens,
                                   int32_t* err_flags, void* workspace, size_t workspace_bytes,
                                   sv_stream_t stream) {
  if (!dtype_ok(dtype)) return SV_EDTYPE;
  if (!(std::isfinite(epsilon) && epsilon >= 0.0 && std::isfinite(delta) && delta >= 0.0)) return SV_EINVAL;
  TreeParams P{};
  size_t smem = 0;
  const sv_status st = tree_setup(P, smem, true, temperature, B, n_nodes, V, dtype, parent, parent_batch_stride,
                                  cand_tokens, target_logits, uniforms, max_depth, accept_len, path_nodes,
                                  out_tokens, err_flags, workspace, workspace_bytes);
  if (st != SV_OK || B == 0) return st;
  P.l2eps = epsilon > 0.0 ? std::log2(epsilon) : -INFINITY;
  P.l2delta = delta > 0.0 ? std::log2(delta) : -INFINITY;
  return dispatch<TypicalLauncher>(dtype, false, P, smem, reinterpret_cast<hipStream_t>(stream));
}

size_t spec_row_stats_workspace(int64_t rows, int64_t V, sv_dtype dtype) {
  if (rows < 0 || V < 1 || !dtype_ok(dtype)) return 0;
  return rowstats_layout(rows, V, dtype).total;
}

sv_status spec_row_stats(sv_dtype dtype, float temperature, int64_t rows, int64_t V, const void* x,
                         float* row_max, float* row_lse, int32_t* row_argmax, int32_t* err_flags,
                         void* workspace, size_t workspace_bytes, sv_stream_t stream) {
  if (!dtype_ok(dtype)) return SV_EDTYPE;
  if (rows < 0 || V < 1 || !temperature_ok(temperature)) return SV_EINVAL;
  if (!shape_ok(V, dtype)) return SV_ELIMIT;
  if (rows == 0) return SV_OK;
  if (!x) return SV_EINVAL;
  const Layout lay = rowstats_layout(rows, V, dtype);
  if (!ws_ok(workspace, workspace_bytes, lay.total)) return SV_EWORKSPACE;
  RowStatsParams P{};
  P.x = static_cast<const char*>(x);
  P.row_max = row_max;
  P.row_lse = row_lse;
  P.row_argmax = row_argmax;
  P.err_flags = err_flags;
  char* ws = static_cast<char*>(workspace);
  P.parts = reinterpret_cast<uint64_t*>(ws + lay.off[0]);
  P.row_cnt = reinterpret_cast<uint32_t*>(ws + lay.off[1]);
  P.rows = rows;
  P.V = V;
  P.C = (int)chunks_per_row(V, dtype);
  P.CP = (P.C + WPB - 1) / WPB * WPB;
  P.c0 = temperature_c0(temperature);
  P.n_stream = rows * P.CP;
  if (P.n_stream > MAX_WAVES) return SV_ELIMIT;
  P.tag = next_tag();
  return dispatch<RowStatsLauncher>(dtype, false, P, reinterpret_cast<hipStream_t>(stream));
}

// Device address of `scratch` on the GPU of `stream` (the current device for the
// null stream), looked up once per device with that device current.
constexpr int STATIC_MAX_DEVICES = 64;
static void* g_scratch_addr[STATIC_MAX_DEVICES];
static std::mutex g_scratch_mu;

static sv_status static_scratch(hipStream_t s, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return SV_EHIP;
  int dev = cur;
  if (s != nullptr && hipStreamGetDevice(s, &dev) != hipSuccess) return SV_EHIP;
  if (dev < 0 || dev >= STATIC_MAX_DEVICES) return SV_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return SV_EHIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) return SV_EHIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return SV_OK;
}

sv_status spec_verify_linear_static(sv_mode mode, float temperature, int64_t B, int64_t k, int64_t V,
                                    sv_dtype dtype, const void* target_logits, const void* draft_logits,
                                    const int32_t* draft_tokens, const float* uniforms, int32_t* accept_len,
                                    int32_t* out_tokens, float* p_target, float* p_draft, int32_t* err_flags,
                                    sv_stream_t stream) {
  // every check that needs no device comes first, so a rejected call touches nothing
  if (!dtype_ok(dtype)) return SV_EDTYPE;
  if (mode != SV_GREEDY && mode != SV_STOCHASTIC) return SV_EINVAL;
  if (B < 0 || k < 0 || V < 1) return SV_EINVAL;
  if (k > SV_MAX_K || !shape_ok(V, dtype)) return SV_ELIMIT;
  if (B == 0) return SV_OK;
  const size_t need = linear_layout(B, k, V, dtype, mode).total;
  if (need > (size_t)SV_MAX_STATIC_WORKSPACE) return SV_ELIMIT;
  LinearParams P{};
  // arguments checked against a stand-in for the array: nothing is launched yet
  sv_status st = linear_setup(P, mode, temperature, B, k, V, dtype, target_logits, draft_logits, draft_tokens,
                              uniforms, accept_len, out_tokens, p_target, p_draft, err_flags,
                              reinterpret_cast<void*>((uintptr_t)256), (size_t)SV_MAX_STATIC_WORKSPACE);
  if (st != SV_OK) return st;
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  st = static_scratch(hs, &ws);
  if (st != SV_OK) return st;
  // the previous call on this GPU normally leaves the region zero; a fill makes the
  // call independent of how that one ended
  st = spec_workspace_clear(ws, need, stream);
  if (st != SV_OK) return st;
  st = linear_setup(P, mode, temperature, B, k, V, dtype, target_logits, draft_logits, draft_tokens, uniforms,
                    accept_len, out_tokens, p_target, p_draft, err_flags, ws, (size_t)SV_MAX_STATIC_WORKSPACE);
  if (st != SV_OK) return st;
  return dispatch<LinearLauncher>(dtype, mode == SV_STOCHASTIC, P, hs);
}

sv_status spec_set_wait_limit(double seconds) {
  if (!(seconds >= 0.0 && seconds <= 60.0)) return SV_EINVAL;
  const uint64_t ticks = (uint64_t)(seconds * 1e8);
  return hipMemcpyToSymbol(HIP_SYMBOL(g_wait_ticks), &ticks, sizeof(ticks)) == hipSuccess ? SV_OK : SV_EHIP;
}

sv_status spec_read_probe(const void* a, size_t a_bytes, const void* b, size_t b_bytes, uint32_t* sink,
                          size_t sink_words, sv_stream_t stream) {
  if ((a_bytes && !a) || (b_bytes && !b)) return SV_EINVAL;
  if ((reinterpret_cast<uintptr_t>(a) & 15u) != 0 || (reinterpret_cast<uintptr_t>(b) & 15u) != 0) return SV_EINVAL;
  const int64_t na = (int64_t)(a_bytes / 16), nb = (int64_t)(b_bytes / 16);
  const int64_t ca = (na + CHUNK_UNITS - 1) / CHUNK_UNITS, cb = (nb + CHUNK_UNITS - 1) / CHUNK_UNITS;
  const int64_t nw = ca + cb;
  if (nw == 0) return SV_OK;
  // the documented bound: one word per started 8 KiB of each buffer
  if (!sink || sink_words < (a_bytes + 8191) / 8192 + (b_bytes + 8191) / 8192) return SV_EINVAL;
  if (nw > MAX_WAVES) return SV_ELIMIT;
  hipLaunchKernelGGL(read_probe_kernel, dim3(blocks_for(nw)), dim3(BLOCK), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(a), na, ca, static_cast<const uint4*>(b), nb, nw, sink);
  return launch_status();
}

sv_status spec_workspace_clear(void* workspace, size_t bytes, sv_stream_t stream) {
  if (bytes == 0) return SV_OK;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 15u) != 0) return SV_EINVAL;
  size_t blocks = (bytes / 16 + BLOCK - 1) / BLOCK;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(clear_kernel, dim3((unsigned)blocks), dim3(BLOCK), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<unsigned char*>(workspace), bytes);
  return launch_status();
}

}  // extern "C"
