// Host side of the smolexp C ABI: configuration and argument checks, the
// weight store (bf16 -> exact fp16 re-encoding), the workspace, the launch
// sequence of one denoising call, and HIP-graph capture and replay of it.
#include "smolexp.h"
#include "smolexp_internal.h"
#include "smolexp_train.h"

#include <math.h>
#include <string.h>

#include <functional>
#include <string>
#include <vector>

using namespace smolexp;

namespace {

struct Mat {
  half_t* w = nullptr;  // blocked layout (t16_off) with ld stored columns
  int ld = 0;
  float scale = 1.f;  // real value = stored fp16 value * scale (a power of two)
  float* rs = nullptr;  // 8-bit weights: w holds E4M3 codes, real value = code value * rs[row]
};

void set_w(GemmArgs& g, const Mat& m) {
  g.W = m.w; g.ldw = m.ld; g.w_scale = m.scale; g.wrs = m.rs;
}

struct LayerDev {
  bool self_attn = false;
  Mat qkv, o, gu, down;
};

// One layer of the prefix language model on the device.
struct LmLayerDev {
  Mat qkv, o, gu, down;
};

// Everything that distinguishes one enqueued call from another.
struct CallKey {
  int velocity_mode;
  int B, P, d;
  float t_single;
  const void* kv;
  const uint8_t* mask;
  const float* x_in;    // noise (denoise) or x (velocity)
  float* out;           // out_actions (denoise) or out_v (velocity)
  const float* prev;
  float* vel;
  float* st;
  int* status;
};

bool same_key(const CallKey& a, const CallKey& b) {
  return a.velocity_mode == b.velocity_mode && a.B == b.B && a.P == b.P && a.d == b.d &&
         a.t_single == b.t_single && a.kv == b.kv && a.mask == b.mask && a.x_in == b.x_in &&
         a.out == b.out && a.prev == b.prev && a.vel == b.vel && a.st == b.st && a.status == b.status;
}

struct GraphEntry {
  CallKey key;
  hipGraphExec_t exec;
  uint64_t last_use;
};

constexpr int kGraphCache = 8;

// Kernel ids of smolexp_time_kernel; PR_LOOP (the whole call) records no launches.
enum ProbeKind { PR_QKV = 0, PR_ATTN_SELF, PR_ATTN_CROSS, PR_O, PR_GU, PR_DOWN, PR_ACTOUT, PR_LOOP, PR_QCROSS, PR_TIN, PR_TOUT,
                 PR_COUNT };

}  // namespace

struct smolexp_handle {
  smolexp_config cfg;
  int device = 0;
  bool loaded = false;
  std::string err;
  float ts[kMaxSteps];
  float dt = 0.f;

  // weights
  void* wmem = nullptr;
  Mat w_tin, w_t2, w_out;   // w_tin: the time MLP's first layer with action_in folded in, [720][32]
  half_t* w_t1e = nullptr;  // W_t1[:, 720:] row-major, fp16 x 2^-s_t1e (read by the prologue)
  float s_t1e = 1.f;
  float *b_t1 = nullptr, *b_t2 = nullptr, *b_out = nullptr;  // b_t1 holds b_t1 + W_t1[:, :720] b_in
  std::vector<LayerDev> layers;

  // workspace: the per-call activations for max_batch queries, then the handle's tables
  void* wsmem = nullptr;
  CallWs ws{};
  float* cvec = nullptr;    // time vectors of the schedule (+ one row for velocity calls)
  int* status_dev = nullptr;  // the status word of calls that do not ask for theirs (kRange* bits)
  float2* rope = nullptr;   // [max_prefix + 50][32] (cos, sin) by position
  double* inv_period = nullptr;

  hipStream_t cap = nullptr;
  std::vector<GraphEntry> graphs;
  // large batches: side streams (default priority) of the query groups, and their
  // fork / join events
  std::vector<hipStream_t> grp_streams;
  std::vector<hipEvent_t> grp_ev;
  uint64_t tick = 0;

  bool have_last = false;
  CallKey last{};
  // launches of the timed kernels in the first step of the last directly enqueued call,
  // one per layer (smolexp_time_kernel replays them)
  struct Probe {
    bool attn;
    bool boundary;  // the step boundary launch: g = action_out's arguments, g2 = the next time_in's
    bool tout;      // ... and g3 = the next time_out's
    GemmArgs g, g2, g3;
    AttnArgs a;
    GemmPlan plan;
    AMode am;
    EMode em;
  };
  bool have_probe = false;
  CallKey probe_key{};
  std::vector<Probe> probes[PR_COUNT];

  // prefix language model (smolexp_prefill)
  void* lmem = nullptr;
  std::vector<LmLayerDev> lm;
  bool lm_loaded = false;
  void* pfmem = nullptr;   // its workspace, grown to the largest B x P seen
  size_t pf_rows = 0;
  float* pf_h = nullptr;
  half_t *pf_h16 = nullptr, *pf_o16 = nullptr, *pf_u16 = nullptr;
  bf16_t* pf_q = nullptr;
  float2* pf_ropeq = nullptr;

  // training step (smolexp_train_step): the manifest as loaded (bf16, row-major), the four
  // biases widened to fp32, and the activation workspace grown to the largest batch seen
  bf16_t* wraw = nullptr;
  float* bias32 = nullptr;
  void* trmem = nullptr;
  int tr_B = 0, tr_P = 0;
  hipStream_t tr_side = nullptr;     // the training step's second stream (default priority)
  std::vector<hipEvent_t> tr_ev;     // its fork/join events
  TrainWs tws{};
};

namespace {

int fail(smolexp_t h, int code, const std::string& msg) {
  if (h) h->err = msg;
  return code;
}

int hip_fail(smolexp_t h, hipError_t e, const char* where) {
  std::string m = std::string(where) + ": " + hipGetErrorString(e);
  return fail(h, SMOLEXP_E_HIP, m);
}

bool check_config(const smolexp_config* c, std::string* why) {
  if (!c) { *why = "config is NULL"; return false; }
  if (c->d_model != kD || c->n_q_heads != kHQ || c->n_kv_heads != kHKV || c->head_dim != kHD ||
      c->ffn != kFFN || c->chunk != kChunk || c->action_dim != kAD) {
    *why = "architecture fields must be d_model 720, 15/5 heads of dim 64, ffn 2048, chunk 50, action_dim 32";
    return false;
  }
  if (c->n_layers < 1 || c->n_layers > kMaxLayers) { *why = "n_layers must be 1..64"; return false; }
  if (c->n_steps < 1 || c->n_steps > kMaxSteps) { *why = "n_steps must be 1..64"; return false; }
  if (c->max_batch < 1 || c->max_batch > 1024) { *why = "max_batch must be 1..1024"; return false; }
  if (c->max_prefix < 1 || c->max_prefix > 4096) { *why = "max_prefix must be 1..4096"; return false; }
  if (c->batch_groups < 0 || c->batch_groups > 8) { *why = "batch_groups must be 0..8"; return false; }
  if (c->weight_format != SMOLEXP_WEIGHTS_FP16 && c->weight_format != SMOLEXP_WEIGHTS_E4M3) {
    *why = "weight_format must be SMOLEXP_WEIGHTS_FP16 or SMOLEXP_WEIGHTS_E4M3";
    return false;
  }
  if (c->weight_format == SMOLEXP_WEIGHTS_E4M3 && c->max_batch > kCrossQMaxBatch) {
    *why = "8-bit weights serve batches of at most 8 queries (max_batch 1..8)";
    return false;
  }
  if (!(c->rope_theta > 0.f) || !(c->rms_eps > 0.f) || !(c->t_min_period > 0.f) ||
      !(c->t_max_period > c->t_min_period) || !isfinite(c->rope_theta) || !isfinite(c->t_max_period)) {
    *why = "rope_theta, rms_eps and 0 < t_min_period < t_max_period must be finite and positive";
    return false;
  }
  return true;
}

size_t layer_count(bool self_attn) {
  size_t n = kD + (size_t)kNQ * kD + (size_t)kD * kNQ + kD + 3 * (size_t)kFFN * kD;
  if (self_attn) n += 2 * (size_t)kNKV * kD;
  return n;
}

// Elements of one layer of the prefix language model (manifest order: norm1.g, q, k, v, o,
// norm2.g, gate, up, down).
size_t lm_layer_count() {
  return kLmD + (size_t)kNQKV * kLmD + (size_t)kLmD * kNQ + kLmD + 3 * (size_t)kLmFFN * kLmD;
}

size_t count_weights(int n_layers) {
  size_t n = (size_t)kD * kAD + kD + (size_t)kD * 2 * kD + kD + (size_t)kD * kD + kD;
  for (int l = 0; l < n_layers; ++l) n += layer_count(l % 2 == 0);
  n += kD + (size_t)kAD * kD + kAD;
  return n;
}

float bf2f(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// Power-of-two exponent s so that max|w| * 2^s lies in [2^14, 2^15): every
// bf16 value (8 significant bits) then maps to an fp16 normal number exactly,
// down to max|w| * 2^-29; smaller values land on fp16's subnormal grid.
int shift_for(float mx) {
  if (!(mx > 0.f) || !isfinite(mx)) return 0;
  int e;
  frexpf(mx, &e);  // mx = f * 2^e, f in [0.5, 1)
  return 15 - e;
}

// OCP 8-bit floating point, E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa bits,
// subnormals, largest finite value 448): the code of the value nearest to v (|v| <= 448),
// ties to even.  The quantum of a magnitude a is 2^(max(floor(log2 a), -6) - 3); a / quantum
// is exact and rounds to an integer n in [0, 16]; n = 16 carries into the next binade through
// the code arithmetic ((exponent field) * 8 + mantissa).
uint8_t e4m3_code(double v) {
  const double a = fabs(v);
  int b = -6;
  if (a > 0) {
    int ex;
    frexp(a, &ex);  // a = f 2^ex, f in [0.5, 1): floor(log2 a) = ex - 1
    b = ex - 1 < -6 ? -6 : ex - 1;
  }
  const int n = (int)nearbyint(ldexp(a, 3 - b));  // round to nearest, ties to even
  const int mag = (b == -6 && n < 8) ? n : (b + 7) * 8 + n - 8;
  return (uint8_t)(mag | ((signbit(v) && mag > 0) ? 0x80 : 0));
}

// Exponent e of a row's scale 2^e: the smallest with max|row| / 2^e <= 448 (so the row's
// largest magnitude lands in (224, 448]).  amax = 448 * 2^k gives exactly k.
int e4m3_row_exp(double amax) {
  int e = ilogb(amax) - 8;  // 448 is in [2^8, 2^9): the answer is this or the next
  if (ldexp(amax, -e) > 448.0) ++e;
  return e;
}

int pick_shift(const std::vector<std::pair<const uint16_t*, size_t>>& parts) {
  float mx = 0.f;
  for (auto& p : parts)
    for (size_t i = 0; i < p.second; ++i) {
      const float v = fabsf(bf2f(p.first[i]));
      if (v > mx) mx = v;
    }
  return shift_for(mx);
}

void to_f16(const uint16_t* src, size_t n, int shift, half_t* dst) {
  const float m = ldexpf(1.f, shift);
  for (size_t i = 0; i < n; ++i) dst[i] = (half_t)(bf2f(src[i]) * m);
}

// Rows rows[0..N) (bf16, K values each, K % 8 == 0) as fp16 * 2^shift in the blocked
// layout with kstore >= K stored columns; dst is zero-filled, so the padding stays zero.
void pack_t16(const std::vector<const uint16_t*>& rows, int K, int kstore, int shift, half_t* dst) {
  const float m = ldexpf(1.f, shift);
  for (size_t n = 0; n < rows.size(); ++n)
    for (int k = 0; k < K; ++k) dst[t16_off((int)n, k, kstore / 8)] = (half_t)(bf2f(rows[n][k]) * m);
}

// A weight that follows an RMSNorm, with the norm's gain g folded into its columns:
// W'[n][k] = W[n][k] * g[k] (exact in fp32: two 8-bit significands), stored like
// pack_t16 with the shift chosen for max |W'| and rounded once to fp16.  Returns the shift.
int pack_t16_gain(const std::vector<const uint16_t*>& rows, int K, int kstore, const uint16_t* gain, half_t* dst) {
  std::vector<float> g(K);
  for (int k = 0; k < K; ++k) g[k] = bf2f(gain[k]);
  float mx = 0.f;
  for (size_t n = 0; n < rows.size(); ++n)
    for (int k = 0; k < K; ++k) mx = fmaxf(mx, fabsf(bf2f(rows[n][k]) * g[k]));
  const int shift = shift_for(mx);
  const float m = ldexpf(1.f, shift);
  for (size_t n = 0; n < rows.size(); ++n)
    for (int k = 0; k < K; ++k) dst[t16_off((int)n, k, kstore / 8)] = (half_t)(bf2f(rows[n][k]) * g[k] * m);
  return shift;
}

// Rows 0..N-1 of a matrix given by row(n, values) (K doubles each) as E4M3 codes in the
// blocked layout with kstore stored columns (dst zero-filled, so the padding is code 0) and
// their scales rs[n] (smolexp_quantize_e4m3_rows, one row at a time).  False if a row
// cannot be quantized.
bool pack_e4m3(int N, int K, int kstore, const std::function<void(int, double*)>& row, uint8_t* dst, float* rs) {
  std::vector<double> v(K);
  std::vector<uint8_t> c(K);
  for (int n = 0; n < N; ++n) {
    row(n, v.data());
    if (smolexp_quantize_e4m3_rows(v.data(), 1, K, c.data(), rs + n) != SMOLEXP_OK) return false;
    for (int k = 0; k < K; ++k) dst[t16_off(n, k, kstore / 8)] = c[k];
  }
  return true;
}

// A row source over bf16 rows (K values each), each value times gain[k] when gain is given
// (the RMSNorm fold; the product of two bf16 values is exact in double).
std::function<void(int, double*)> bf16_rows(std::vector<const uint16_t*> rows, int K, const uint16_t* gain = nullptr) {
  return [rows, K, gain](int n, double* out) {
    for (int k = 0; k < K; ++k) out[k] = (double)bf2f(rows[n][k]) * (gain ? (double)bf2f(gain[k]) : 1.0);
  };
}

// Row pointers of a row-major [N][ld] bf16 matrix, starting at column c0.
std::vector<const uint16_t*> rows_of(const uint16_t* p, int N, int ld, int c0 = 0) {
  std::vector<const uint16_t*> r(N);
  for (int n = 0; n < N; ++n) r[n] = p + (size_t)n * ld + c0;
  return r;
}

// Rows of a layer's [Q; K; V] projection ([960 or 1600][K], V absent for cross layers) in
// the order the kernels use: inside each Q and K head, 16-row block q holds dims q*8..q*8+7
// then 32+q*8..32+q*8+7, so the rotation pairs (d, d + 32) share an MFMA tile.
std::vector<const uint16_t*> rope_paired_rows(const uint16_t* pq, const uint16_t* pk, const uint16_t* pv, int K) {
  const bool kv = pk != nullptr;
  const int nrows = kv ? kNQKV : kNQ, rot_heads = kv ? kHQ + kHKV : kHQ;
  std::vector<const uint16_t*> row_src(nrows);
  for (int r = 0; r < kNQ; ++r) row_src[r] = pq + (size_t)r * K;
  if (kv) {
    for (int r = 0; r < kNKV; ++r) row_src[kNQ + r] = pk + (size_t)r * K;
    for (int r = 0; r < kNKV; ++r) row_src[kNQ + kNKV + r] = pv + (size_t)r * K;
  }
  std::vector<const uint16_t*> perm(nrows);
  for (int r = 0; r < nrows; ++r) {
    const int head = r / kHD, rr = r % kHD;
    int src = r;
    if (head < rot_heads) {
      const int q = rr / 16, e = rr % 16;
      src = head * kHD + (e < 8 ? q * 8 + e : kHD / 2 + q * 8 + (e - 8));
    }
    perm[r] = row_src[src];
  }
  return perm;
}

// Rows of the [gate; up] projection ([2 F][K]) interleaved in 16-row blocks: block j holds
// gate rows 8j..8j+7, then up rows 8j..8j+7 (the SwiGLU epilogue pairs them).
std::vector<const uint16_t*> gate_up_rows(const uint16_t* pg, const uint16_t* pu, int F, int K) {
  std::vector<const uint16_t*> gu(2 * (size_t)F);
  for (int j = 0; j < F / 8; ++j)
    for (int e = 0; e < 8; ++e) {
      gu[16 * j + e] = pg + (size_t)(8 * j + e) * K;
      gu[16 * j + 8 + e] = pu + (size_t)(8 * j + e) * K;
    }
  return gu;
}

int round16(int n) { return (n + 15) & ~15; }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

struct CallArgs {
  bool velocity;
  const void* kv;
  const uint8_t* mask;
  int P;
  const float* x_in;
  float* out;
  int B;
  const float* prev;
  int d;
  float* vel;
  float* st;
  float t_single;
  int* status;  // the caller's status word, or nullptr (the handle's)
};

CallKey key_of(const CallArgs& c) {
  CallKey k;
  memset(&k, 0, sizeof(k));
  k.velocity_mode = c.velocity;
  k.B = c.B; k.P = c.P; k.d = c.d; k.t_single = c.velocity ? c.t_single : 0.f;
  k.kv = c.kv; k.mask = c.mask; k.x_in = c.x_in; k.out = c.out; k.prev = c.prev; k.vel = c.vel; k.st = c.st;
  k.status = c.status;
  return k;
}

// Queries per group of a call (the groups' loops run concurrently): `batch_groups` groups
// when the config sets it, else two groups from 64 queries on and one per 64 queries from 192
// on; every group but the last holds a multiple of 8 queries (whole 16-row blocks of the
// blocked operands).  Measured (16 layers, 10 steps, ms per call, one group / two / three /
// four): batch 64 at prefix 257 16.65 / 15.25 / 18.0 / 21.0; batch 96 21.2 / 20.3 / 21.3; batch
// 128 at prefix 177 27.0 / 24.0 / 26.4 / 26.7; batch 32 11.1 / 11.8; batch 24 10.0 / 11.0;
// batch 16 8.70 / 8.92.  Returns the count.
constexpr int kMaxGroups = 8;
int group_sizes(const smolexp_config& cfg, int B, int* sz) {
  int G = cfg.batch_groups > 0 ? cfg.batch_groups : (B >= 192 ? B / 64 : B >= 64 ? 2 : 1);
  G = G < kMaxGroups ? G : kMaxGroups;
  auto base_of = [&](int g) { return ((B + g - 1) / g + 7) / 8 * 8; };
  int base = base_of(G);
  while (G > 1 && (G - 1) * base >= B) base = base_of(--G);
  for (int i = 0; i < G - 1; ++i) sz[i] = base;
  sz[G - 1] = B - (G - 1) * base;
  return G;
}

int ensure_group_streams(smolexp_t h, int G) {
  while ((int)h->grp_streams.size() < G - 1) {
    hipStream_t st = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess)
      return fail(h, SMOLEXP_E_HIP, "group stream creation failed");
    h->grp_streams.push_back(st);
  }
  while ((int)h->grp_ev.size() < G) {
    hipEvent_t ev = nullptr;
    if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess)
      return fail(h, SMOLEXP_E_HIP, "group event creation failed");
    h->grp_ev.push_back(ev);
  }
  return SMOLEXP_OK;
}

// The launch sequence of one call, on the per-call workspace w.  may_fork = false keeps
// every launch on s (one group), as the no-alloc entry point needs.
int enqueue(smolexp_t h, const CallArgs& c, const CallWs& w, hipStream_t s, bool record_probes,
            bool may_fork = true) {
  const int B = c.B, P = c.P, L = h->cfg.n_layers;
  const int n_t = c.velocity ? 1 : h->cfg.n_steps;
  // time vectors: the schedule's were computed when the weights were loaded; a velocity
  // call computes its own (one t) into the row after them
  float* const cvec = c.velocity ? h->cvec + (size_t)kMaxSteps * kD : h->cvec;
  hipError_t e;
  if (record_probes) {
    for (int i = 0; i < PR_COUNT; ++i) h->probes[i].clear();
    h->probe_key = key_of(c);
    h->have_probe = true;
  }

  // the call's status word: cleared by the prologue, kRange* bits set by any kernel that rounds
  // an activation beyond fp16's range
  int* const status = c.status ? c.status : h->status_dev;
  PrologueArgs pa;
  memset(&pa, 0, sizeof(pa));
  pa.status = status;
  pa.B = B;
  pa.n_t = c.velocity ? 1 : 0;
  pa.t[0] = c.t_single;
  pa.mask = c.mask;
  pa.P = P;
  pa.rope = h->rope;
  pa.ropeq = w.ropeq;
  pa.x_in = c.x_in;
  pa.x = w.x;
  pa.w_t1e = h->w_t1e;
  pa.s_t1 = h->s_t1e;
  pa.b_t1 = h->b_t1;
  pa.cvec = cvec;
  pa.inv_period = h->inv_period;
  if ((e = launch_prologue(pa, s)) != hipSuccess) return hip_fail(h, e, "prologue launch");

  const size_t kvLayer = (size_t)2 * B * kHKV * (size_t)P * kHD;  // elements per layer
  const bf16_t* kv = static_cast<const bf16_t*>(c.kv);
  bool first_step = true;  // probes are recorded in the first step only
  auto record = [&](int probe, const GemmPlan& plan, AMode am, EMode em, const GemmArgs& g) {
    if (record_probes && first_step && probe >= 0) {
      smolexp_handle::Probe p;
      memset(&p, 0, sizeof(p));
      p.attn = false; p.g = g; p.plan = plan; p.am = am; p.em = em;
      h->probes[probe].push_back(p);
    }
  };

  // The loop of one group of queries: rows b0 * 50 .. (b0 + Bg) * 50 - 1 of every workspace
  // buffer (b0 is a multiple of 8, so the blocked operands start on a 16-row block), the
  // group's slices of the prefix cache, mask, noise and outputs, on stream gs.
  auto run_group = [&](int b0, int Bg, hipStream_t gs) -> int {
    const int Mg = Bg * kChunk, r0 = b0 * kChunk;
    CallWs wg = w;
    wg.x = w.x + (size_t)r0 * kAD;
    wg.h = w.h + (size_t)r0 * kD;
    wg.s16 = w.s16 + (size_t)r0 * kD;
    wg.o16 = w.o16 + (size_t)r0 * kNQ;
    wg.u16 = w.u16 + (size_t)r0 * kFFN;
    wg.h16 = w.h16 + (size_t)r0 * kKPad;
    wg.q = w.q + (size_t)r0 * kNQ;
    wg.kc = w.kc + (size_t)r0 * kNKV;
    wg.vc = w.vc + (size_t)r0 * kNKV;
    wg.ropeq = w.ropeq + (size_t)r0 * (kHD / 2);
    wg.x2 = w.x2 + (size_t)r0 * kAD;
    const size_t qOff = (size_t)r0 * kAD;                        // [b][50][32] arrays
    const size_t kvOff = (size_t)b0 * kHKV * (size_t)P * kHD;    // inside each layer's K and V
    const uint8_t* mask_g = c.mask + (size_t)b0 * P;
    // every projection: the planned kernel (plan_for); RMSNorm'd projections (Q/K/V,
    // gate/up, action_out) read h16 = fp16(h), over the zero-padded K = 768 on the pipelined GEMM
    auto gemm = [&](int probe, AMode am, EMode em, const GemmArgs& g0) -> hipError_t {
      GemmArgs g = g0;
      if (am == A_NORM) { g.A = wg.h16; g.lda = kKPad; }
      const GemmPlan plan = plan_for(g.M, g.N, g.K, am, em, g.wrs != nullptr);
      if (plan.kind == 2) {
        if (am == A_NORM) g.K = kKPad;
        record(probe, plan, am, em, g);
        return launch_gemm_big(plan, em, am == A_NORM, g, gs);
      }
      record(probe, plan, am, em, g);
      return launch_gemm(plan, am, em, g, gs);
    };
    auto norm_gemm = [&](int probe, EMode em, const GemmArgs& g) -> hipError_t { return gemm(probe, A_NORM, em, g); };
    hipError_t e;
    GemmArgs g;
    memset(&g, 0, sizeof(g));
    g.status = status;
    g.M = Mg;
    g.inv_k = 1.0f / kD;
    g.eps = h->cfg.rms_eps;
    // action_in + time MLP, first layer, of step k: s = SiLU(W_t1[:, :720] (W_in x + b_in) +
    // W_t1[:, 720:] e(t) + b_t1), computed as (W_t1[:, :720] W_in) x + the step's time vector
    // (whose bias holds W_t1[:, :720] b_in); the prefix overwrite is applied to x as it is read
    // and stored back into the state.
    // Where action_out takes the register-resident K split (up to 4800 rows), the end of step k
    // and the start of step k + 1 run as one launch (both are row-local; at 3200 rows that launch
    // takes 7.2 us against 9.0 for action_out alone, batch 128 23.21 -> 23.03 ms), and
    // the Euler state of step k lives in x (k even) or x2 (k odd); otherwise always in x.
    const bool w8 = h->w_out.rs != nullptr;
    const bool fuse_boundary = plan_for(Mg, kAD, kD, A_NORM, E_ACTOUT, w8).kind == 0;
    auto state = [&](int k) { return fuse_boundary && (k & 1) ? wg.x2 : wg.x; };
    // one query (50 rows): the boundary launch also runs the time MLP's second layer of step k + 1
    // (every workgroup holds the 16 rows' whole hidden layer in LDS)
    const bool fuse_time_out = fuse_boundary && Mg <= kBoundaryTimeOutMaxRows;
    auto time_out_args = [&]() {
      GemmArgs go = g;
      go.N = kD; go.K = kD; go.A = wg.s16; go.lda = kD;
      set_w(go, h->w_t2); go.bias = h->b_t2;
      go.h = wg.h; go.h16 = wg.h16;
      return go;
    };
    auto time_in_args = [&](int k) {
      GemmArgs gt = g;
      gt.N = kD; gt.K = kAD; gt.A = state(k); gt.lda = kAD;
      gt.x = state(k); gt.noise = c.x_in + qOff; gt.prev = c.prev ? c.prev + (size_t)b0 * c.d * kAD : nullptr;
      gt.ow_rows = c.velocity ? 0 : c.d; gt.t = c.velocity ? c.t_single : h->ts[k];
      set_w(gt, h->w_tin); gt.bias = cvec + (size_t)k * kD;
      gt.out16 = wg.s16; gt.ldo = kD;
      return gt;
    };
    for (int k = 0; k < n_t; ++k) {
      first_step = k == 0;

      // time MLP: the first layer (unless the previous step's boundary launch ran it), then
      // h = W_t2 s + b_t2
      if (k == 0 || !fuse_boundary) {
        if ((e = gemm(PR_TIN, A_X, E_TIMEIN, time_in_args(k))) != hipSuccess) return hip_fail(h, e, "time_in launch");
      }

      if (k == 0 || !fuse_time_out) {
        if ((e = gemm(PR_TOUT, A_F16, E_H_BIAS, time_out_args())) != hipSuccess) return hip_fail(h, e, "time_out launch");
      }

      for (int l = 0; l < L; ++l) {
        const LayerDev& ld = h->layers[l];
        // cross layers of a small batch: the Q projection runs inside the attention launch
        const bool fold_q = !ld.self_attn && use_cross_q(Bg);
        if (!fold_q) {
          GemmArgs gq = g;
          gq.N = ld.self_attn ? kNQKV : kNQ; gq.K = kD;
          set_w(gq, ld.qkv);
          gq.q = wg.q; gq.kc = wg.kc; gq.vc = wg.vc; gq.ropeq = wg.ropeq;
          if ((e = norm_gemm(ld.self_attn ? PR_QKV : PR_QCROSS, E_QKV, gq)) != hipSuccess) return hip_fail(h, e, "qkv launch");
        }

        AttnArgs aa;
        memset(&aa, 0, sizeof(aa));
        aa.status = status;
        aa.q = wg.q; aa.kc = wg.kc; aa.vc = wg.vc;
        aa.pk = kv + (size_t)l * kvLayer + kvOff;
        aa.pv = kv + (size_t)l * kvLayer + kvLayer / 2 + kvOff;
        aa.mask = mask_g; aa.out = wg.o16; aa.B = Bg; aa.P = P;
        if (fold_q) {
          aa.wq = ld.qkv.w; aa.ldw = ld.qkv.ld; aa.w_scale = ld.qkv.scale; aa.wrs = ld.qkv.rs;
          aa.h16 = wg.h16; aa.inv_k = g.inv_k; aa.eps = g.eps; aa.ropeq = wg.ropeq;
        }
        const int pr = ld.self_attn ? PR_ATTN_SELF : PR_ATTN_CROSS;
        if (record_probes && first_step) {
          smolexp_handle::Probe p;
          memset(&p, 0, sizeof(p));
          p.attn = true; p.a = aa;
          h->probes[pr].push_back(p);
        }
        if ((e = launch_attention(ld.self_attn, aa, gs)) != hipSuccess) return hip_fail(h, e, "attention launch");

        GemmArgs gop = g;
        gop.N = kD; gop.K = kNQ; gop.A = wg.o16; gop.lda = kNQ;
        set_w(gop, ld.o); gop.h = wg.h; gop.h16 = wg.h16;
        if ((e = gemm(PR_O, A_F16, E_H_RESID, gop)) != hipSuccess) return hip_fail(h, e, "o launch");

        GemmArgs gg = g;
        gg.N = kGU; gg.K = kD;
        set_w(gg, ld.gu); gg.out16 = wg.u16; gg.ldo = kFFN;
        if ((e = norm_gemm(PR_GU, E_SWIGLU, gg)) != hipSuccess) return hip_fail(h, e, "gate/up launch");

        GemmArgs gd = g;
        gd.N = kD; gd.K = kFFN; gd.A = wg.u16; gd.lda = kFFN;
        set_w(gd, ld.down); gd.h = wg.h; gd.h16 = wg.h16;
        if ((e = gemm(PR_DOWN, A_F16, E_H_RESID, gd)) != hipSuccess) return hip_fail(h, e, "down launch");
      }

      // final RMSNorm + action_out; Euler update x += dt v
      GemmArgs gv = g;
      gv.N = kAD; gv.K = kD;
      set_w(gv, h->w_out); gv.bias = h->b_out;
      gv.x = state(k); gv.dt = h->dt;
      const size_t stepElems = (size_t)B * kChunk * kAD;
      if (c.velocity) {
        gv.vel_out = c.out + qOff;
      } else {
        gv.vel_out = c.vel ? c.vel + (size_t)k * stepElems + qOff : nullptr;
        gv.st_out = c.st ? c.st + (size_t)k * stepElems + qOff : nullptr;
        gv.final_out = (k == n_t - 1) ? c.out + qOff : nullptr;
      }
      if (fuse_boundary && k + 1 < n_t) {
        gv.A = wg.h16; gv.lda = kKPad;
        const GemmArgs gt = time_in_args(k + 1), go = time_out_args();
        if (record_probes && first_step) {
          smolexp_handle::Probe p;
          memset(&p, 0, sizeof(p));
          p.boundary = true; p.tout = fuse_time_out; p.g = gv; p.g2 = gt; p.g3 = go;
          h->probes[PR_ACTOUT].push_back(p);
        }
        if ((e = launch_step_boundary(gv, gt, fuse_time_out ? &go : nullptr, gs)) != hipSuccess)
          return hip_fail(h, e, "step boundary launch");
      } else if ((e = norm_gemm(PR_ACTOUT, E_ACTOUT, gv)) != hipSuccess) {
        return hip_fail(h, e, "action_out launch");
      }
    }
    return SMOLEXP_OK;
  };

  // Large batches run as groups of queries whose loops are independent chains of launches:
  // the groups after the first fork onto side streams after the prologue (parallel branches
  // of the captured graph) and join the call's stream at the end, so each group's launches
  // fill the CUs that another group's launch leaves idle.
  int gsz[kMaxGroups];
  int G = group_sizes(h->cfg, B, gsz);
  if (!may_fork) {
    G = 1;
    gsz[0] = B;
  }
  if (G > 1) {
    const int rc0 = ensure_group_streams(h, G);
    if (rc0 != SMOLEXP_OK) return rc0;
    if ((e = hipEventRecord(h->grp_ev[0], s)) != hipSuccess) return hip_fail(h, e, "group fork");
    for (int gi = 1; gi < G; ++gi)
      if ((e = hipStreamWaitEvent(h->grp_streams[gi - 1], h->grp_ev[0], 0)) != hipSuccess) return hip_fail(h, e, "group fork");
  }
  int rc = SMOLEXP_OK;
  for (int gi = 0, b0 = 0; gi < G && rc == SMOLEXP_OK; b0 += gsz[gi], ++gi)
    rc = run_group(b0, gsz[gi], gi == 0 ? s : h->grp_streams[gi - 1]);
  // join every side stream, also after an error, so no group outlives the call's stream
  for (int gi = 1; gi < G; ++gi) {
    hipError_t ej = hipEventRecord(h->grp_ev[gi], h->grp_streams[gi - 1]);
    if (ej == hipSuccess) ej = hipStreamWaitEvent(s, h->grp_ev[gi], 0);
    if (ej != hipSuccess && rc == SMOLEXP_OK) rc = hip_fail(h, ej, "group join");
  }
  return rc;
}

void drop_graphs(smolexp_t h) {
  for (auto& g : h->graphs) (void)hipGraphExecDestroy(g.exec);
  h->graphs.clear();
}

// Replays the cached graph of `key`, or captures enq's launches into a new one (least
// recently used evicted beyond kGraphCache) and launches it on s.
template <class Enq>
int run_cached(smolexp_t h, const CallKey& key, hipStream_t s, Enq enq) {
  for (auto& g : h->graphs) {
    if (same_key(g.key, key)) {
      g.last_use = ++h->tick;
      hipError_t e = hipGraphLaunch(g.exec, s);
      if (e != hipSuccess) return hip_fail(h, e, "hipGraphLaunch");
      return SMOLEXP_OK;
    }
  }
  hipError_t e = hipStreamBeginCapture(h->cap, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return hip_fail(h, e, "hipStreamBeginCapture");
  const int rc = enq(h->cap);
  hipGraph_t graph = nullptr;
  e = hipStreamEndCapture(h->cap, &graph);
  if (rc != SMOLEXP_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    return rc;
  }
  if (e != hipSuccess) return hip_fail(h, e, "hipStreamEndCapture");
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  (void)hipGraphDestroy(graph);
  if (e != hipSuccess) return hip_fail(h, e, "hipGraphInstantiate");
  if ((int)h->graphs.size() >= kGraphCache) {
    size_t lru = 0;
    for (size_t i = 1; i < h->graphs.size(); ++i)
      if (h->graphs[i].last_use < h->graphs[lru].last_use) lru = i;
    // the evicted graph may still be running on a caller's stream
    (void)hipStreamSynchronize(s);
    (void)hipGraphExecDestroy(h->graphs[lru].exec);
    h->graphs.erase(h->graphs.begin() + lru);
  }
  h->graphs.push_back(GraphEntry{key, exec, ++h->tick});
  e = hipGraphLaunch(exec, s);
  if (e != hipSuccess) return hip_fail(h, e, "hipGraphLaunch");
  return SMOLEXP_OK;
}

int run_call(smolexp_t h, const CallArgs& c, hipStream_t s) {
  const CallKey key = key_of(c);
  h->last = key;
  h->have_last = true;
  if (!h->cfg.use_graphs) return enqueue(h, c, h->ws, s, true);
  return run_cached(h, key, s, [&](hipStream_t cs) { return enqueue(h, c, h->ws, cs, true); });
}

int check_call(smolexp_t h, const void* kv, const uint8_t* mask, int P, const float* x_in, float* out, int B) {
  if (!h) return SMOLEXP_E_INVAL;
  h->err.clear();
  if (!h->loaded) return fail(h, SMOLEXP_E_STATE, "weights are not loaded");
  if (!kv || !mask || !x_in || !out) return fail(h, SMOLEXP_E_INVAL, "a required pointer is NULL");
  if (B < 1 || B > h->cfg.max_batch) return fail(h, SMOLEXP_E_INVAL, "batch out of range 1..max_batch");
  if (P < 1 || P > h->cfg.max_prefix) return fail(h, SMOLEXP_E_INVAL, "prefix_len out of range 1..max_prefix");
  return SMOLEXP_OK;
}

// Grow the prefill workspace to hold `rows` = B P rows (synchronous; blocked operands are
// padded to whole 16-row blocks).
int ensure_prefill_workspace(smolexp_t h, size_t rows) {
  if (rows <= h->pf_rows) return SMOLEXP_OK;
  if (h->pfmem) {
    (void)hipDeviceSynchronize();
    (void)hipFree(h->pfmem);
    h->pfmem = nullptr;
    h->pf_rows = 0;
  }
  const size_t rp = (rows + 15) & ~(size_t)15;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  const size_t o_h = take(rp * kLmD * 4), o_h16 = take(rp * kLmD * 2), o_q = take(rows * kNQ * 2);
  const size_t o_o = take(rp * kNQ * 2), o_u = take(rp * kLmFFN * 2), o_rq = take(rows * (kHD / 2) * sizeof(float2));
  hipError_t e = hipMalloc(&h->pfmem, off);
  if (e != hipSuccess) return fail(h, SMOLEXP_E_NOMEM, "prefill workspace allocation failed");
  char* base = static_cast<char*>(h->pfmem);
  h->pf_h = (float*)(base + o_h);
  h->pf_h16 = (half_t*)(base + o_h16);
  h->pf_q = (bf16_t*)(base + o_q);
  h->pf_o16 = (half_t*)(base + o_o);
  h->pf_u16 = (half_t*)(base + o_u);
  h->pf_ropeq = (float2*)(base + o_rq);
  h->pf_rows = rows;
  return SMOLEXP_OK;
}

// The launch sequence of one prefill: per layer, RMSNorm'd Q/K/V with RoPE (K and V straight
// into the cache), and for every layer but the last the prefix self-attention, o, gate/up
// and down.
int enqueue_prefill(smolexp_t h, const bf16_t* emb, const uint8_t* mask, int P, bf16_t* kv, int B, hipStream_t s) {
  const int L = h->cfg.n_layers, M = B * P;
  hipError_t e;
  PrefillPrologueArgs pp;
  memset(&pp, 0, sizeof(pp));
  pp.status = h->status_dev;
  pp.B = B; pp.P = P; pp.emb = emb; pp.mask = mask; pp.rope = h->rope;
  pp.h = h->pf_h; pp.h16 = h->pf_h16; pp.ropeq = h->pf_ropeq;
  if ((e = launch_prefill_prologue(pp, s)) != hipSuccess) return hip_fail(h, e, "prefill prologue launch");
  auto gemm = [&](AMode am, EMode em, const GemmArgs& g) -> hipError_t {
    const GemmPlan plan = plan_prefill(g.M, g.N, g.K, em);
    if (plan.kind == 2) return launch_gemm_big(plan, em, am == A_NORM, g, s);
    return launch_gemm(plan, am, em, g, s);
  };
  const size_t kvLayer = (size_t)2 * B * kHKV * (size_t)P * kHD;
  for (int l = 0; l < L; ++l) {
    const LmLayerDev& ld = h->lm[l];
    bf16_t* kcache = kv + (size_t)l * kvLayer;
    bf16_t* vcache = kcache + kvLayer / 2;
    GemmArgs g;
    memset(&g, 0, sizeof(g));
    g.status = h->status_dev;
    g.M = M;
    g.inv_k = 1.0f / kLmD;
    g.eps = h->cfg.rms_eps;

    GemmArgs gq = g;
    gq.N = kNQKV; gq.K = kLmD; gq.A = h->pf_h16; gq.lda = kLmD;
    set_w(gq, ld.qkv);
    gq.q = h->pf_q; gq.kc = kcache; gq.vc = vcache; gq.seq = P; gq.ropeq = h->pf_ropeq;
    if ((e = gemm(A_NORM, E_PF_QKV, gq)) != hipSuccess) return hip_fail(h, e, "prefill qkv launch");
    if (l == L - 1) break;  // the last layer's keys and values are all the cache needs

    AttnArgs aa;
    memset(&aa, 0, sizeof(aa));
    aa.status = h->status_dev;
    aa.q = h->pf_q; aa.pk = kcache; aa.pv = vcache; aa.mask = mask; aa.out = h->pf_o16;
    aa.B = B; aa.P = P; aa.seq = P;
    if ((e = launch_prefix_attention(aa, s)) != hipSuccess) return hip_fail(h, e, "prefill attention launch");

    GemmArgs go = g;
    go.N = kLmD; go.K = kNQ; go.A = h->pf_o16; go.lda = kNQ;
    set_w(go, ld.o); go.h = h->pf_h; go.h16 = h->pf_h16;
    if ((e = gemm(A_F16, E_PF_RESID, go)) != hipSuccess) return hip_fail(h, e, "prefill o launch");

    GemmArgs gg = g;
    gg.N = kLmGU; gg.K = kLmD; gg.A = h->pf_h16; gg.lda = kLmD;
    set_w(gg, ld.gu); gg.out16 = h->pf_u16; gg.ldo = kLmFFN;
    if ((e = gemm(A_NORM, E_SWIGLU, gg)) != hipSuccess) return hip_fail(h, e, "prefill gate/up launch");

    GemmArgs gd = g;
    gd.N = kLmD; gd.K = kLmFFN; gd.A = h->pf_u16; gd.lda = kLmFFN;
    set_w(gd, ld.down); gd.h = h->pf_h; gd.h16 = h->pf_h16;
    if ((e = gemm(A_F16, E_PF_RESID, gd)) != hipSuccess) return hip_fail(h, e, "prefill down launch");
  }
  return SMOLEXP_OK;
}

}  // namespace

extern "C" {

void smolexp_default_config(smolexp_config* c) {
  if (!c) return;
  memset(c, 0, sizeof(*c));
  c->n_layers = 16;
  c->d_model = kD;
  c->n_q_heads = kHQ;
  c->n_kv_heads = kHKV;
  c->head_dim = kHD;
  c->ffn = kFFN;
  c->chunk = kChunk;
  c->action_dim = kAD;
  c->n_steps = 10;
  c->max_batch = 128;
  c->max_prefix = 512;
  c->rope_theta = 10000.f;
  c->rms_eps = 1e-6f;
  c->t_min_period = 4e-3f;
  c->t_max_period = 4.0f;
  c->use_graphs = 1;
}

size_t smolexp_weight_count(const smolexp_config* cfg) {
  std::string why;
  if (!check_config(cfg, &why)) return 0;
  return count_weights(cfg->n_layers);
}

int smolexp_batch_groups(const smolexp_config* cfg, int batch, int* sizes) {
  std::string why;
  if (!check_config(cfg, &why) || batch < 1 || batch > cfg->max_batch) return SMOLEXP_E_INVAL;
  int sz[kMaxGroups];
  const int G = group_sizes(*cfg, batch, sz);
  if (sizes)
    for (int i = 0; i < G; ++i) sizes[i] = sz[i];
  return G;
}

int smolexp_quantize_e4m3_rows(const double* w, int rows, int cols, uint8_t* codes, float* scales) {
  if (rows < 0 || cols < 0) return SMOLEXP_E_INVAL;
  if (rows > 0 && (!scales || (cols > 0 && (!w || !codes)))) return SMOLEXP_E_INVAL;
  for (int r = 0; r < rows; ++r) {
    const double* row = w + (size_t)r * cols;
    double amax = 0.0;
    for (int k = 0; k < cols; ++k) {
      if (!isfinite(row[k])) return SMOLEXP_E_INVAL;
      amax = fmax(amax, fabs(row[k]));
    }
    int e = 0;
    if (amax > 0) {
      e = e4m3_row_exp(amax);
      if (e < -126 || e > 127) return SMOLEXP_E_INVAL;  // the scale must be a normal float
    }
    scales[r] = ldexpf(1.f, e);
    for (int k = 0; k < cols; ++k) codes[(size_t)r * cols + k] = e4m3_code(ldexp(row[k], -e));
  }
  return SMOLEXP_OK;
}

int smolexp_schedule(const smolexp_config* cfg, float* t_out, float* dt_out) {
  std::string why;
  if (!check_config(cfg, &why) || !t_out) return SMOLEXP_E_INVAL;
  const float dt = (float)(-1.0 / (double)cfg->n_steps);
  volatile float t = 1.0f;  // each step rounds to fp32
  for (int k = 0; k < cfg->n_steps; ++k) {
    t_out[k] = t;
    t = t + dt;
  }
  if (dt_out) *dt_out = dt;
  return SMOLEXP_OK;
}

int smolexp_create(const smolexp_config* cfg, int hip_device, smolexp_t* out) {
  std::string why;
  if (!out) return SMOLEXP_E_INVAL;
  if (!check_config(cfg, &why)) return SMOLEXP_E_INVAL;
  if (hip_device < 0) return SMOLEXP_E_INVAL;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || hip_device >= ndev) return SMOLEXP_E_HIP;
  if (hipSetDevice(hip_device) != hipSuccess) return SMOLEXP_E_HIP;

  smolexp_t h = new (std::nothrow) smolexp_handle();
  if (!h) return SMOLEXP_E_NOMEM;
  h->cfg = *cfg;
  h->device = hip_device;
  smolexp_schedule(cfg, h->ts, &h->dt);

  const size_t Mpad = (size_t)round16(cfg->max_batch * kChunk);  // blocked operands hold whole 16-row blocks
  const int n_pos = cfg->max_prefix + kChunk;
  size_t off = call_ws_bytes(cfg->max_batch);
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  const size_t o_cv = take((size_t)(kMaxSteps + 1) * kD * 4);  // the schedule's time vectors + one for velocity calls
  const size_t o_rope = take((size_t)n_pos * (kHD / 2) * sizeof(float2));
  const size_t o_invp = take((size_t)(kD / 2) * sizeof(double));
  const size_t o_status = take(sizeof(int));
  // the no-alloc entry point's fixed workspace on this device: its address, looked up once
  char* scratch_base = nullptr;
  size_t scratch_bytes = 0;
  if (noalloc_scratch(hip_device, &scratch_base, &scratch_bytes) != hipSuccess) { delete h; return SMOLEXP_E_HIP; }
  hipError_t e = hipMalloc(&h->wsmem, off);
  if (e != hipSuccess) { delete h; return SMOLEXP_E_NOMEM; }
  char* base = static_cast<char*>(h->wsmem);
  h->ws = carve_call_ws(base, cfg->max_batch);
  h->cvec = (float*)(base + o_cv);
  h->rope = (float2*)(base + o_rope);
  h->inv_period = (double*)(base + o_invp);
  h->status_dev = (int*)(base + o_status);

  e = hipStreamCreateWithFlags(&h->cap, hipStreamNonBlocking);
  // the columns 720..767 of h16 are read by the K = 768 GEMM and never written: zero them once
  if (e == hipSuccess) e = hipMemsetAsync(h->ws.h16, 0, Mpad * kKPad * 2, h->cap);
  if (e == hipSuccess) e = launch_rope_table(h->rope, n_pos, cfg->rope_theta, h->cap);
  if (e == hipSuccess) e = launch_inv_period_table(h->inv_period, cfg->t_min_period, cfg->t_max_period, h->cap);
  if (e == hipSuccess) e = hipStreamSynchronize(h->cap);
  if (e != hipSuccess) {
    smolexp_destroy(h);
    return SMOLEXP_E_HIP;
  }
  *out = h;
  return SMOLEXP_OK;
}

int smolexp_load_weights(smolexp_t h, const uint16_t* src, size_t n_elems) {
  if (!h) return SMOLEXP_E_INVAL;
  h->err.clear();
  if (!src) return fail(h, SMOLEXP_E_INVAL, "weight buffer is NULL");
  const int L = h->cfg.n_layers;
  if (n_elems != count_weights(L)) return fail(h, SMOLEXP_E_SIZE, "weight count does not match the manifest");
  if (hipSetDevice(h->device) != hipSuccess) return fail(h, SMOLEXP_E_HIP, "hipSetDevice failed");

  // Device layout: fp16 GEMM matrices in the blocked layout (gate/up interleaved in 16-row
  // blocks, Q/K rows permuted per head; Q/K/V and gate/up with K padded to 768 for the
  // large-M GEMM; the RMSNorm gains folded into Q/K/V, gate/up and action_out), the
  // time-embedding half of W_t1 row-major for the prologue, fp32 biases.  With 8-bit weights
  // the streamed matrices hold E4M3 codes at the same element offsets (one byte each), and
  // each has an fp32 scale per stored row.
  const bool w8 = h->cfg.weight_format == SMOLEXP_WEIGHTS_E4M3;
  const size_t eb = w8 ? 1 : 2;  // bytes per streamed weight element
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  const size_t o_wtin = take((size_t)kD * kAD * eb), o_wt1e = take((size_t)kD * kD * 2);
  const size_t o_wt2 = take((size_t)kD * kD * eb);
  const size_t o_bt1 = take(kD * 4), o_bt2 = take(kD * 4);
  std::vector<size_t> o_qkv(L), o_o(L), o_gu(L), o_dn(L);
  for (int l = 0; l < L; ++l) {
    o_qkv[l] = take((size_t)(l % 2 == 0 ? kNQKV : kNQ) * kKPad * eb);
    o_o[l] = take((size_t)kD * kNQ * eb);
    o_gu[l] = take((size_t)kGU * kKPad * eb);
    o_dn[l] = take((size_t)kD * kFFN * eb);
  }
  const size_t o_wout = take((size_t)kAD * kD * eb), o_bout = take(kAD * 4);
  // row scales of the 8-bit matrices (every row count here is a multiple of 16)
  size_t r_tin = 0, r_t2 = 0, r_out = 0;
  std::vector<size_t> r_qkv(L, 0), r_o(L, 0), r_gu(L, 0), r_dn(L, 0);
  if (w8) {
    r_tin = take(kD * 4); r_t2 = take(kD * 4); r_out = take(kAD * 4);
    for (int l = 0; l < L; ++l) {
      r_qkv[l] = take((size_t)(l % 2 == 0 ? kNQKV : kNQ) * 4);
      r_o[l] = take(kD * 4);
      r_gu[l] = take(kGU * 4);
      r_dn[l] = take(kD * 4);
    }
  }
  std::vector<char> hostbuf;
  try {
    hostbuf.assign(off, 0);
  } catch (...) {
    return fail(h, SMOLEXP_E_NOMEM, "host staging allocation failed");
  }
  char* hb = hostbuf.data();

  size_t pos = 0;
  auto next = [&](size_t n) { const uint16_t* p = src + pos; pos += n; return p; };
  auto vec32 = [&](const uint16_t* p, size_t n, size_t o) {
    float* d = (float*)(hb + o);
    for (size_t i = 0; i < n; ++i) d[i] = bf2f(p[i]);
  };
  Mat w_tin, w_t2, w_out;
  std::vector<LayerDev> layers(L);
  std::vector<int> sh_qkv(L), sh_o(L), sh_gu(L), sh_dn(L);

  const uint16_t* p_win = next((size_t)kD * kAD);
  const uint16_t* p_bin = next(kD);
  const uint16_t* p_wt1 = next((size_t)kD * 2 * kD);
  const uint16_t* p_bt1 = next(kD);
  const uint16_t* p_wt2 = next((size_t)kD * kD);
  const uint16_t* p_bt2 = next(kD);
  int s;
  // action_in feeds only the action half of the time MLP's first layer, a linear map:
  // W_t1[:, :720] (W_in x + b_in) = (W_t1[:, :720] W_in) x + W_t1[:, :720] b_in.  The
  // [720][32] product and the bias term depend on the weights alone, so they are formed
  // here once (fp64 sums of the bf16 values; the product rounded once to fp16) and the
  // layer reads the Euler state directly.
  {
    std::vector<double> win((size_t)kD * kAD), bin(kD), acc(kAD);
    for (size_t i = 0; i < win.size(); ++i) win[i] = bf2f(p_win[i]);
    for (int i = 0; i < kD; ++i) bin[i] = bf2f(p_bin[i]);
    std::vector<float> wtin((size_t)kD * kAD);
    std::vector<double> wtin_d(w8 ? (size_t)kD * kAD : 0);
    float* bt1 = (float*)(hb + o_bt1);
    float mx = 0.f;
    for (int j = 0; j < kD; ++j) {
      const uint16_t* wr = p_wt1 + (size_t)j * 2 * kD;  // row j, columns 0..719: the action half
      std::fill(acc.begin(), acc.end(), 0.0);
      double bsum = bf2f(p_bt1[j]);
      for (int i = 0; i < kD; ++i) {
        const double w = bf2f(wr[i]);
        const double* ir = win.data() + (size_t)i * kAD;
        for (int c = 0; c < kAD; ++c) acc[c] += w * ir[c];
        bsum += w * bin[i];
      }
      for (int c = 0; c < kAD; ++c) {
        wtin[(size_t)j * kAD + c] = (float)acc[c];
        mx = fmaxf(mx, fabsf((float)acc[c]));
        if (w8) wtin_d[(size_t)j * kAD + c] = acc[c];
      }
      bt1[j] = (float)bsum;
    }
    if (w8) {  // the double product, quantized once
      const double* wd = wtin_d.data();
      if (!pack_e4m3(kD, kAD, kAD, [wd](int n, double* o) { memcpy(o, wd + (size_t)n * kAD, kAD * sizeof(double)); },
                     (uint8_t*)(hb + o_wtin), (float*)(hb + r_tin)))
        return fail(h, SMOLEXP_E_INVAL, "a weight row cannot take an 8-bit row scale (largest magnitude at most 448 x 2^-127)");
    } else {
      s = shift_for(mx);
      const float m = ldexpf(1.f, s);
      half_t* dst = (half_t*)(hb + o_wtin);
      for (int j = 0; j < kD; ++j)
        for (int c = 0; c < kAD; ++c) dst[t16_off(j, c, kAD / 8)] = (half_t)(wtin[(size_t)j * kAD + c] * m);
      w_tin.scale = ldexpf(1.f, -s);
    }
    w_tin.ld = kAD;
  }
  bool q_ok = true;  // every 8-bit row quantized
  auto q8 = [&](int N, int K, int kstore, const std::function<void(int, double*)>& row, size_t o, size_t r) {
    q_ok = q_ok && pack_e4m3(N, K, kstore, row, (uint8_t*)(hb + o), (float*)(hb + r));
  };
  // the time-embedding half, row-major for the prologue, with a scale of its own
  std::vector<std::pair<const uint16_t*, size_t>> t1e_rows(kD);
  for (int j = 0; j < kD; ++j) t1e_rows[j] = {p_wt1 + (size_t)j * 2 * kD + kD, (size_t)kD};
  s = pick_shift(t1e_rows);
  for (int j = 0; j < kD; ++j) to_f16(t1e_rows[j].first, kD, s, (half_t*)(hb + o_wt1e) + (size_t)j * kD);
  const float s_t1e = ldexpf(1.f, -s);
  if (w8) {
    q8(kD, kD, kD, bf16_rows(rows_of(p_wt2, kD, kD), kD), o_wt2, r_t2);
  } else {
    s = pick_shift({{p_wt2, (size_t)kD * kD}});
    pack_t16(rows_of(p_wt2, kD, kD), kD, kD, s, (half_t*)(hb + o_wt2));
    w_t2.scale = ldexpf(1.f, -s);
  }
  w_t2.ld = kD;
  vec32(p_bt2, kD, o_bt2);

  for (int l = 0; l < L; ++l) {
    const bool self_attn = l % 2 == 0;
    LayerDev& ld = layers[l];
    ld.self_attn = self_attn;
    const uint16_t* g1 = next(kD);
    const uint16_t* pq = next((size_t)kNQ * kD);
    const uint16_t* pk = self_attn ? next((size_t)kNKV * kD) : nullptr;
    const uint16_t* pvv = self_attn ? next((size_t)kNKV * kD) : nullptr;
    const uint16_t* po = next((size_t)kD * kNQ);
    const uint16_t* g2 = next(kD);
    const uint16_t* pg = next((size_t)kFFN * kD);
    const uint16_t* pu = next((size_t)kFFN * kD);
    const uint16_t* pd = next((size_t)kD * kFFN);
    // q, k, v are consecutive in the manifest: one [1600, 720] matrix (or q alone)
    ld.qkv.ld = kKPad; ld.o.ld = kNQ; ld.gu.ld = kKPad; ld.down.ld = kFFN;
    if (w8) {
      q8(self_attn ? kNQKV : kNQ, kD, kKPad, bf16_rows(rope_paired_rows(pq, pk, pvv, kD), kD, g1), o_qkv[l], r_qkv[l]);
      q8(kD, kNQ, kNQ, bf16_rows(rows_of(po, kD, kNQ), kNQ), o_o[l], r_o[l]);
      q8(kGU, kD, kKPad, bf16_rows(gate_up_rows(pg, pu, kFFN, kD), kD, g2), o_gu[l], r_gu[l]);
      q8(kD, kFFN, kFFN, bf16_rows(rows_of(pd, kD, kFFN), kFFN), o_dn[l], r_dn[l]);
      continue;
    }
    s = pack_t16_gain(rope_paired_rows(pq, pk, pvv, kD), kD, kKPad, g1, (half_t*)(hb + o_qkv[l]));
    ld.qkv.scale = ldexpf(1.f, -s);
    s = pick_shift({{po, (size_t)kD * kNQ}});
    pack_t16(rows_of(po, kD, kNQ), kNQ, kNQ, s, (half_t*)(hb + o_o[l]));
    ld.o.scale = ldexpf(1.f, -s);
    s = pack_t16_gain(gate_up_rows(pg, pu, kFFN, kD), kD, kKPad, g2, (half_t*)(hb + o_gu[l]));
    ld.gu.scale = ldexpf(1.f, -s);
    s = pick_shift({{pd, (size_t)kD * kFFN}});
    pack_t16(rows_of(pd, kD, kFFN), kFFN, kFFN, s, (half_t*)(hb + o_dn[l]));
    ld.down.scale = ldexpf(1.f, -s);
  }
  const uint16_t* p_gf = next(kD);
  const uint16_t* p_wout = next((size_t)kAD * kD);
  const uint16_t* p_bout = next(kAD);
  if (w8) {
    q8(kAD, kD, kD, bf16_rows(rows_of(p_wout, kAD, kD), kD, p_gf), o_wout, r_out);
  } else {
    s = pack_t16_gain(rows_of(p_wout, kAD, kD), kD, kD, p_gf, (half_t*)(hb + o_wout));
    w_out.scale = ldexpf(1.f, -s);
  }
  w_out.ld = kD;
  vec32(p_bout, kAD, o_bout);
  if (!q_ok) return fail(h, SMOLEXP_E_INVAL, "a weight row cannot take an 8-bit row scale (largest magnitude at most 448 x 2^-127)");

  if (h->wmem) {
    (void)hipDeviceSynchronize();
    (void)hipFree(h->wmem);
    h->wmem = nullptr;
    h->loaded = false;
  }
  drop_graphs(h);
  h->have_last = false;
  hipError_t e = hipMalloc(&h->wmem, off);
  if (e != hipSuccess) return fail(h, SMOLEXP_E_NOMEM, "device weight allocation failed");
  e = hipMemcpy(h->wmem, hb, off, hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(h, e, "weight upload");
  char* db = static_cast<char*>(h->wmem);
  w_tin.w = (half_t*)(db + o_wtin); w_t2.w = (half_t*)(db + o_wt2); w_out.w = (half_t*)(db + o_wout);
  h->w_tin = w_tin; h->w_t2 = w_t2; h->w_out = w_out;
  h->w_t1e = (half_t*)(db + o_wt1e);
  h->s_t1e = s_t1e;
  h->b_t1 = (float*)(db + o_bt1); h->b_t2 = (float*)(db + o_bt2);
  h->b_out = (float*)(db + o_bout);
  for (int l = 0; l < L; ++l) {
    layers[l].qkv.w = (half_t*)(db + o_qkv[l]);
    layers[l].o.w = (half_t*)(db + o_o[l]);
    layers[l].gu.w = (half_t*)(db + o_gu[l]);
    layers[l].down.w = (half_t*)(db + o_dn[l]);
  }
  if (w8) {
    h->w_tin.rs = (float*)(db + r_tin); h->w_t2.rs = (float*)(db + r_t2); h->w_out.rs = (float*)(db + r_out);
    for (int l = 0; l < L; ++l) {
      layers[l].qkv.rs = (float*)(db + r_qkv[l]);
      layers[l].o.rs = (float*)(db + r_o[l]);
      layers[l].gu.rs = (float*)(db + r_gu[l]);
      layers[l].down.rs = (float*)(db + r_dn[l]);
    }
  }
  h->layers = layers;
  // the time vectors of the schedule: W_t1[:, 720:] e(t_k) + b_t1 depends on the weights
  // and the fixed flow times only, so it is computed here once, not in every call
  PrologueArgs pa;
  memset(&pa, 0, sizeof(pa));
  pa.B = 0;
  pa.n_t = h->cfg.n_steps;
  for (int k = 0; k < pa.n_t; ++k) pa.t[k] = h->ts[k];
  pa.w_t1e = h->w_t1e;
  pa.s_t1 = h->s_t1e;
  pa.b_t1 = h->b_t1;
  pa.cvec = h->cvec;
  pa.inv_period = h->inv_period;
  e = launch_prologue(pa, h->cap);
  if (e == hipSuccess) e = hipStreamSynchronize(h->cap);
  if (e != hipSuccess) return hip_fail(h, e, "time vectors");
  // the training step reads the manifest as given, plus its biases in fp32
  if (!h->wraw) {
    if (hipMalloc(&h->wraw, n_elems * 2) != hipSuccess) return fail(h, SMOLEXP_E_NOMEM, "weight copy allocation failed");
    if (hipMalloc(&h->bias32, (3 * kD + kAD) * sizeof(float)) != hipSuccess)
      return fail(h, SMOLEXP_E_NOMEM, "bias copy allocation failed");
  }
  {
    TrOffsets to;
    train_offsets(L, 0, &to);
    std::vector<float> b32(3 * kD + kAD);
    auto widen = [&](size_t off, int n, float* dst) {
      for (int i = 0; i < n; ++i) {
        const uint32_t u = (uint32_t)src[off + i] << 16;
        memcpy(&dst[i], &u, 4);
      }
    };
    widen(to.ain_b, kD, b32.data());
    widen(to.tin_b, kD, b32.data() + kD);
    widen(to.tout_b, kD, b32.data() + 2 * kD);
    widen(to.aout_b, kAD, b32.data() + 3 * kD);
    e = hipMemcpy(h->wraw, src, n_elems * 2, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(h->bias32, b32.data(), b32.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(h, e, "weight copy upload");
  }
  h->loaded = true;
  return SMOLEXP_OK;
}

size_t smolexp_lm_weight_count(const smolexp_config* cfg) {
  std::string why;
  if (!check_config(cfg, &why)) return 0;
  return (size_t)cfg->n_layers * lm_layer_count();
}

int smolexp_load_lm_weights(smolexp_t h, const uint16_t* bf16_host, size_t n_elems) {
  if (!h) return SMOLEXP_E_INVAL;
  h->err.clear();
  if (!bf16_host) return fail(h, SMOLEXP_E_INVAL, "weights pointer is NULL");
  const int L = h->cfg.n_layers;
  if (n_elems != (size_t)L * lm_layer_count())
    return fail(h, SMOLEXP_E_SIZE, "weight count does not match the language model's manifest");
  if (hipSetDevice(h->device) != hipSuccess) return fail(h, SMOLEXP_E_HIP, "hipSetDevice failed");
  const uint16_t* src = bf16_host;
  // device layout per layer: [Q; K; V] rope-paired with norm1's gain folded, o, gate/up
  // interleaved with norm2's gain folded, down; all fp16 blocked, K stored as is (960 and
  // 2560 are multiples of 64)
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  std::vector<size_t> o_qkv(L), o_o(L), o_gu(L), o_dn(L);
  for (int l = 0; l < L; ++l) {
    o_qkv[l] = take((size_t)kNQKV * kLmD * 2);
    o_o[l] = take((size_t)kLmD * kNQ * 2);
    o_gu[l] = take((size_t)kLmGU * kLmD * 2);
    o_dn[l] = take((size_t)kLmD * kLmFFN * 2);
  }
  std::vector<char> hostbuf;
  try {
    hostbuf.assign(off, 0);
  } catch (...) {
    return fail(h, SMOLEXP_E_NOMEM, "host staging allocation failed");
  }
  char* hb = hostbuf.data();
  size_t pos = 0;
  auto next = [&](size_t n) { const uint16_t* p = src + pos; pos += n; return p; };
  std::vector<LmLayerDev> layers(L);
  for (int l = 0; l < L; ++l) {
    LmLayerDev& ld = layers[l];
    const uint16_t* g1 = next(kLmD);
    const uint16_t* pq = next((size_t)kNQ * kLmD);
    const uint16_t* pk = next((size_t)kNKV * kLmD);
    const uint16_t* pv = next((size_t)kNKV * kLmD);
    const uint16_t* po = next((size_t)kLmD * kNQ);
    const uint16_t* g2 = next(kLmD);
    const uint16_t* pg = next((size_t)kLmFFN * kLmD);
    const uint16_t* pu = next((size_t)kLmFFN * kLmD);
    const uint16_t* pd = next((size_t)kLmD * kLmFFN);
    int s = pack_t16_gain(rope_paired_rows(pq, pk, pv, kLmD), kLmD, kLmD, g1, (half_t*)(hb + o_qkv[l]));
    ld.qkv.scale = ldexpf(1.f, -s); ld.qkv.ld = kLmD;
    s = pick_shift({{po, (size_t)kLmD * kNQ}});
    pack_t16(rows_of(po, kLmD, kNQ), kNQ, kNQ, s, (half_t*)(hb + o_o[l]));
    ld.o.scale = ldexpf(1.f, -s); ld.o.ld = kNQ;
    s = pack_t16_gain(gate_up_rows(pg, pu, kLmFFN, kLmD), kLmD, kLmD, g2, (half_t*)(hb + o_gu[l]));
    ld.gu.scale = ldexpf(1.f, -s); ld.gu.ld = kLmD;
    s = pick_shift({{pd, (size_t)kLmD * kLmFFN}});
    pack_t16(rows_of(pd, kLmD, kLmFFN), kLmFFN, kLmFFN, s, (half_t*)(hb + o_dn[l]));
    ld.down.scale = ldexpf(1.f, -s); ld.down.ld = kLmFFN;
  }
  if (h->lmem) {
    (void)hipDeviceSynchronize();
    (void)hipFree(h->lmem);
    h->lmem = nullptr;
    h->lm_loaded = false;
  }
  hipError_t e = hipMalloc(&h->lmem, off);
  if (e != hipSuccess) return fail(h, SMOLEXP_E_NOMEM, "device weight allocation failed");
  e = hipMemcpy(h->lmem, hb, off, hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(h, e, "weight upload");
  char* db = static_cast<char*>(h->lmem);
  for (int l = 0; l < L; ++l) {
    layers[l].qkv.w = (half_t*)(db + o_qkv[l]);
    layers[l].o.w = (half_t*)(db + o_o[l]);
    layers[l].gu.w = (half_t*)(db + o_gu[l]);
    layers[l].down.w = (half_t*)(db + o_dn[l]);
  }
  h->lm = layers;
  h->lm_loaded = true;
  return SMOLEXP_OK;
}

int smolexp_prefill(smolexp_t h, const void* prefix_emb, const uint8_t* prefix_mask, int prefix_len,
                    void* out_kv, int batch, void* hip_stream) {
  if (!h) return SMOLEXP_E_INVAL;
  h->err.clear();
  if (!h->lm_loaded) return fail(h, SMOLEXP_E_STATE, "language-model weights are not loaded");
  if (!prefix_emb || !prefix_mask || !out_kv) return fail(h, SMOLEXP_E_INVAL, "a required pointer is NULL");
  if (batch < 1 || batch > h->cfg.max_batch) return fail(h, SMOLEXP_E_INVAL, "batch out of range 1..max_batch");
  if (prefix_len < 1 || prefix_len > h->cfg.max_prefix)
    return fail(h, SMOLEXP_E_INVAL, "prefix_len out of range 1..max_prefix");
  if (hipSetDevice(h->device) != hipSuccess) return fail(h, SMOLEXP_E_HIP, "hipSetDevice failed");
  const int rc = ensure_prefill_workspace(h, (size_t)batch * prefix_len);
  if (rc != SMOLEXP_OK) return rc;
  return enqueue_prefill(h, static_cast<const bf16_t*>(prefix_emb), prefix_mask, prefix_len,
                         static_cast<bf16_t*>(out_kv), batch, static_cast<hipStream_t>(hip_stream));
}

int smolexp_train_step(smolexp_t h, const void* prefix_kv, const uint8_t* prefix_mask, int prefix_len,
                       const float* actions, const float* noise, const float* t, float* out_grads, float* out_loss,
                       int batch, void* hip_stream) {
  if (!h) return SMOLEXP_E_INVAL;
  h->err.clear();
  if (!h->loaded) return fail(h, SMOLEXP_E_STATE, "weights are not loaded");
  if (!prefix_kv || !prefix_mask || !actions || !noise || !t || !out_grads || !out_loss)
    return fail(h, SMOLEXP_E_INVAL, "a required pointer is NULL");
  if (batch < 1 || batch > h->cfg.max_batch) return fail(h, SMOLEXP_E_INVAL, "batch out of range 1..max_batch");
  if (prefix_len < 1 || prefix_len > h->cfg.max_prefix)
    return fail(h, SMOLEXP_E_INVAL, "prefix_len out of range 1..max_prefix");
  if (hipSetDevice(h->device) != hipSuccess) return fail(h, SMOLEXP_E_HIP, "hipSetDevice failed");
  const int L = h->cfg.n_layers;
  if (batch > h->tr_B || prefix_len > h->tr_P) {
    const int nb = batch > h->tr_B ? batch : h->tr_B, np = prefix_len > h->tr_P ? prefix_len : h->tr_P;
    if (h->trmem) {
      (void)hipDeviceSynchronize();
      drop_graphs(h);
      (void)hipFree(h->trmem);
      h->trmem = nullptr;
      h->tr_B = h->tr_P = 0;
    }
    if (hipMalloc(&h->trmem, train_workspace_bytes(nb, np, L)) != hipSuccess)
      return fail(h, SMOLEXP_E_NOMEM, "training workspace allocation failed");
    h->tr_B = nb;
    h->tr_P = np;
  }
  if (!h->tr_side) {
    if (hipStreamCreateWithFlags(&h->tr_side, hipStreamNonBlocking) != hipSuccess)
      return fail(h, SMOLEXP_E_HIP, "training side stream creation failed");
    h->tr_ev.assign(8 * kMaxLayers, nullptr);
    for (auto& ev : h->tr_ev)
      if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess)
        return fail(h, SMOLEXP_E_HIP, "training event creation failed");
  }
  TrainArgs ta;
  memset(&ta, 0, sizeof(ta));
  ta.side = h->tr_side;
  ta.ev = h->tr_ev.data();
  ta.n_ev = (int)h->tr_ev.size();
  ta.B = batch; ta.P = prefix_len; ta.L = L;
  ta.kv = static_cast<const bf16_t*>(prefix_kv); ta.mask = prefix_mask;
  ta.actions = actions; ta.noise = noise; ta.t = t; ta.grads = out_grads; ta.loss = out_loss;
  ta.w = h->wraw; ta.bias32 = h->bias32; ta.rope = h->rope; ta.inv_period = h->inv_period;
  ta.rms_eps = h->cfg.rms_eps;
  // the workspace is carved for this call's batch and prefix length (it holds at least that)
  train_carve(static_cast<char*>(h->trmem), batch, prefix_len, L, &ta.ws);
  ta.split_cap = train_split_cap(batch);
  const hipStream_t st = static_cast<hipStream_t>(hip_stream);
  auto enq = [&](hipStream_t cs) -> int {
    const hipError_t e = train_enqueue(ta, cs);
    return e == hipSuccess ? SMOLEXP_OK : hip_fail(h, e, "training step launch");
  };
  if (!h->cfg.use_graphs) return enq(st);
  // one graph per call signature, as for the denoiser (velocity_mode 2 marks a training step;
  // the graphs hold the workspace's addresses, so growing it drops them)
  CallKey key;
  memset(&key, 0, sizeof(key));
  key.velocity_mode = 2;
  key.B = batch; key.P = prefix_len;
  key.kv = prefix_kv; key.mask = prefix_mask; key.x_in = noise; key.prev = actions;
  key.out = out_grads; key.vel = out_loss; key.st = const_cast<float*>(t);
  return run_cached(h, key, st, enq);
}

int smolexp_denoise_ex(smolexp_t h, const void* prefix_kv, const uint8_t* prefix_mask, int prefix_len,
                       const float* noise, float* out_actions, int batch, void* hip_stream,
                       const smolexp_denoise_opts* opts) {
  int rc = check_call(h, prefix_kv, prefix_mask, prefix_len, noise, out_actions, batch);
  if (rc != SMOLEXP_OK) return rc;
  CallArgs c;
  memset(&c, 0, sizeof(c));
  c.velocity = false;
  c.kv = prefix_kv; c.mask = prefix_mask; c.P = prefix_len; c.x_in = noise; c.out = out_actions; c.B = batch;
  if (opts) {
    if (opts->overwrite_rows < 0 || opts->overwrite_rows > kChunk)
      return fail(h, SMOLEXP_E_INVAL, "overwrite_rows out of range 0..50");
    if (opts->overwrite_rows > 0 && !opts->prev_actions)
      return fail(h, SMOLEXP_E_INVAL, "overwrite_rows > 0 needs prev_actions");
    c.d = opts->overwrite_rows;
    c.prev = c.d > 0 ? opts->prev_actions : nullptr;
    c.vel = opts->out_velocities;
    c.st = opts->out_states;
    c.status = opts->out_status;
  }
  if (hipSetDevice(h->device) != hipSuccess) return fail(h, SMOLEXP_E_HIP, "hipSetDevice failed");
  return run_call(h, c, static_cast<hipStream_t>(hip_stream));
}

int smolexp_denoise(smolexp_t h, const void* prefix_kv, const uint8_t* prefix_mask, int prefix_len,
                    const float* noise, float* out_actions, int batch, void* hip_stream) {
  return smolexp_denoise_ex(h, prefix_kv, prefix_mask, prefix_len, noise, out_actions, batch, hip_stream, nullptr);
}

int smolexp_denoise_noalloc(smolexp_t h, const void* prefix_kv, const uint8_t* prefix_mask, int prefix_len,
                            const float* noise, float* out_actions, int batch, void* hip_stream) {
  int rc = check_call(h, prefix_kv, prefix_mask, prefix_len, noise, out_actions, batch);
  if (rc != SMOLEXP_OK) return rc;
  if (batch > kNoAllocMaxBatch)
    return fail(h, SMOLEXP_E_INVAL, "batch above the no-alloc workspace's maximum of 16 queries");
  if (hipSetDevice(h->device) != hipSuccess) return fail(h, SMOLEXP_E_HIP, "hipSetDevice failed");
  char* base = nullptr;
  size_t bytes = 0;
  hipError_t e = noalloc_scratch(h->device, &base, &bytes);
  if (e != hipSuccess) return hip_fail(h, e, "no-alloc workspace lookup");
  const CallWs w = carve_call_ws(base, kNoAllocMaxBatch);
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  // the array keeps the last call's contents: the zero columns of h16 are cleared each call
  e = launch_zero_h16_pad(w.h16, round16(batch * kChunk), s);
  if (e != hipSuccess) return hip_fail(h, e, "no-alloc workspace clear");
  CallArgs c;
  memset(&c, 0, sizeof(c));
  c.velocity = false;
  c.kv = prefix_kv; c.mask = prefix_mask; c.P = prefix_len; c.x_in = noise; c.out = out_actions; c.B = batch;
  return enqueue(h, c, w, s, false, false);
}

int smolexp_velocity(smolexp_t h, const void* prefix_kv, const uint8_t* prefix_mask, int prefix_len,
                     const float* x, float t, float* out_v, int batch, void* hip_stream) {
  int rc = check_call(h, prefix_kv, prefix_mask, prefix_len, x, out_v, batch);
  if (rc != SMOLEXP_OK) return rc;
  if (!isfinite(t)) return fail(h, SMOLEXP_E_INVAL, "t must be finite");
  CallArgs c;
  memset(&c, 0, sizeof(c));
  c.velocity = true;
  c.kv = prefix_kv; c.mask = prefix_mask; c.P = prefix_len; c.x_in = x; c.out = out_v; c.B = batch; c.t_single = t;
  if (hipSetDevice(h->device) != hipSuccess) return fail(h, SMOLEXP_E_HIP, "hipSetDevice failed");
  return run_call(h, c, static_cast<hipStream_t>(hip_stream));
}

int smolexp_time_kernel(smolexp_t h, int kernel, int reps, void* hip_stream, float* avg_us) {
  if (!h) return SMOLEXP_E_INVAL;
  h->err.clear();
  if (!avg_us || reps < 1 || reps > 100000 || kernel < 0 || kernel >= PR_COUNT)
    return fail(h, SMOLEXP_E_INVAL, "bad kernel id, reps or avg_us");
  if (!h->have_last) return fail(h, SMOLEXP_E_STATE, "no previous denoise call to time");
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  CallArgs lastc;
  memset(&lastc, 0, sizeof(lastc));
  {
    const CallKey& k = h->last;
    lastc.velocity = k.velocity_mode; lastc.kv = k.kv; lastc.mask = k.mask; lastc.P = k.P; lastc.x_in = k.x_in;
    lastc.out = k.out; lastc.B = k.B; lastc.prev = k.prev; lastc.d = k.d; lastc.vel = k.vel; lastc.st = k.st;
    lastc.t_single = k.t_single;
    lastc.status = k.status;
  }
  if (kernel != PR_LOOP && (!h->have_probe || !same_key(h->probe_key, h->last))) {
    // the previous call was a graph replay of another key: enqueue it once directly to get its launches
    int rc0 = enqueue(h, lastc, h->ws, s, true);
    if (rc0 != SMOLEXP_OK) return rc0;
  }
  if (kernel != PR_LOOP && h->probes[kernel].empty()) return fail(h, SMOLEXP_E_STATE, "kernel not part of the previous call");
  // launch i replays the (i mod n)-th recorded instance: every layer's weights in turn, as in the loop
  auto launch = [&](int i, hipStream_t st) -> hipError_t {
    const std::vector<smolexp_handle::Probe>& v = h->probes[kernel];
    const smolexp_handle::Probe& p = v[(size_t)i % v.size()];
    if (p.attn) return launch_attention(kernel == PR_ATTN_SELF, p.a, st);
    if (p.boundary) return launch_step_boundary(p.g, p.g2, p.tout ? &p.g3 : nullptr, st);
    if (p.plan.kind == 2) return launch_gemm_big(p.plan, p.em, p.am == A_NORM, p.g, st);
    return launch_gemm(p.plan, p.am, p.em, p.g, st);
  };
  hipGraphExec_t exec = nullptr;
  if (kernel != PR_LOOP && h->cfg.use_graphs) {
    // one graph of `reps` launches (the loop itself runs as a graph)
    hipError_t e = hipStreamBeginCapture(h->cap, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) return hip_fail(h, e, "hipStreamBeginCapture");
    hipError_t el = hipSuccess;
    for (int i = 0; i < reps && el == hipSuccess; ++i) el = launch(i, h->cap);
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(h->cap, &graph);
    if (el != hipSuccess || e != hipSuccess) {
      if (graph) (void)hipGraphDestroy(graph);
      return hip_fail(h, el != hipSuccess ? el : e, "kernel timing capture");
    }
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) return hip_fail(h, e, "kernel timing graph");
    e = hipGraphLaunch(exec, s);  // untimed pass
    if (e != hipSuccess) {
      (void)hipStreamSynchronize(s);
      (void)hipGraphExecDestroy(exec);
      return hip_fail(h, e, "kernel timing graph launch");
    }
  }
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (exec) { (void)hipStreamSynchronize(s); (void)hipGraphExecDestroy(exec); }
    return fail(h, SMOLEXP_E_HIP, "hipEventCreate");
  }
  hipError_t e = hipEventRecord(e0, s);
  int rc = SMOLEXP_OK;
  if (exec) {
    if (e == hipSuccess) e = hipGraphLaunch(exec, s);
  } else {
    for (int i = 0; i < reps && e == hipSuccess && rc == SMOLEXP_OK; ++i) {
      if (kernel == PR_LOOP) rc = run_call(h, lastc, s);  // the whole loop: replay the previous call
      else e = launch(i, s);
    }
  }
  if (e == hipSuccess) e = hipEventRecord(e1, s);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (exec) {
    (void)hipStreamSynchronize(s);
    (void)hipGraphExecDestroy(exec);
  }
  if (rc != SMOLEXP_OK) return rc;
  if (e != hipSuccess) return hip_fail(h, e, "kernel timing");
  *avg_us = ms * 1000.f / reps;
  return SMOLEXP_OK;
}

const char* smolexp_strerror(int code) {
  switch (code) {
    case SMOLEXP_OK: return "ok";
    case SMOLEXP_E_INVAL: return "invalid argument";
    case SMOLEXP_E_STATE: return "call out of order";
    case SMOLEXP_E_SIZE: return "wrong weight count";
    case SMOLEXP_E_NOMEM: return "out of memory";
    case SMOLEXP_E_HIP: return "HIP runtime error";
    default: return "unknown error code";
  }
}

const char* smolexp_last_error(smolexp_t h) { return h ? h->err.c_str() : ""; }

void smolexp_destroy(smolexp_t h) {
  if (!h) return;
  (void)hipSetDevice(h->device);
  (void)hipDeviceSynchronize();
  drop_graphs(h);
  if (h->cap) (void)hipStreamDestroy(h->cap);
  for (auto st : h->grp_streams) (void)hipStreamDestroy(st);
  for (auto ev : h->grp_ev) (void)hipEventDestroy(ev);
  if (h->wmem) (void)hipFree(h->wmem);
  if (h->wsmem) (void)hipFree(h->wsmem);
  if (h->lmem) (void)hipFree(h->lmem);
  if (h->pfmem) (void)hipFree(h->pfmem);
  if (h->trmem) (void)hipFree(h->trmem);
  for (auto ev : h->tr_ev)
    if (ev) (void)hipEventDestroy(ev);
  if (h->tr_side) (void)hipStreamDestroy(h->tr_side);
  if (h->wraw) (void)hipFree(h->wraw);
  if (h->bias32) (void)hipFree(h->bias32);
  delete h;
}

}  // extern "C"
