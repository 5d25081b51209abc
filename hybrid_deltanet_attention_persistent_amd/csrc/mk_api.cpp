// mk_api.cpp -- host side of the C ABI declared in include/mk.h: validation, arena
// layout, weight re-tiling, state reset and the persistent-kernel launches.
//
// Validation of a call (config, tensors, sizes, context length, call order) is
// finished before the first HIP call of that call, so every rejection is
// side-effect free and can be exercised without a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "mk.h"
#include "mk_layout.h"

extern "C" hipError_t mk_launch_forward(const MkLaunch *a, int ncol_template, int variant, hipStream_t stream);
extern "C" hipError_t mk_forward_occupancy(int ncol_template, int variant, int *blocks_per_cu);
extern "C" hipError_t mk_static_scratch(void **ptr);
extern "C" hipError_t mk_prefill_enqueue(const MkDev *d, const MkLayerDev *layers_host, const MkPf *pf,
                                         const int32_t *tokens, int n, int32_t *argmax, float *logits,
                                         hipStream_t st, hipStream_t side, hipEvent_t *ev, int max_blocks,
                                         const MkPfW *pfw);

static thread_local std::string g_err;

static int fail(int code, const std::string &msg) {
  g_err = msg;
  return code;
}

#define HIPCHECK(expr)                                                                        \
  do {                                                                                        \
    hipError_t e_ = (expr);                                                                   \
    if (e_ != hipSuccess) return fail(MK_EHIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

static const uint32_t MK_MAGIC = 0x6d6b4d44u;

struct mk_model {
  uint32_t magic;
  int device;
  mk_config cfg;
  std::vector<uint8_t> kinds;
  MkDev dev;                            // the selected sequence's view (state, KV cache, control words)
  std::vector<MkLayerDev> layers_host;  // its layer table (host copy) for the prefill driver
  // sequences (mk_config.n_seq): each has its own layer table (shared weights, own state and
  // KV cache) and control block; calls other than mk_decode_batch act on the selected one
  int cur = 0;
  std::vector<MkDev> seq_dev;
  std::vector<std::vector<MkLayerDev>> seq_layers_host;
  std::vector<int32_t> seq_pos_hi;      // per sequence: upper bound of its device position
  std::vector<uint8_t> seq_verified;    // per sequence: its last forward was a verify (updates may be pending)
  MkPf pf;                              // prefill scratch
  std::vector<MkPfW> pfw;               // per layer: prefill copies of the projection weights
  char *arena;
  size_t arena_bytes;
  uint2 *xch;                           // exchange slots of mk_decode_step (in the arena)
  uint2 *static_xch;                    // device address of the static slots (mk_decode_step_static)
  int32_t *gen;                         // [64] device buffers of mk_generate_lookup (in the arena)
  // regions cleared by mk_reset_state
  std::vector<std::pair<size_t, size_t>> state_regions;
  int32_t pos_hi;  // the selected sequence's upper bound of the device position (exact unless a verify ran)
  uint32_t tag;    // next exchange tag
  // prefill in two row blocks: the second block's kernels run on a side stream (created on first
  // use, default priority), ordered against the caller's stream by events (n_layers + 2)
  int pf_blocks = 2;
  hipStream_t pf_side = nullptr;
  std::vector<hipEvent_t> pf_ev;
};

// ------------------------------------------------------------------------------ layout
namespace {

struct Region {
  size_t off = 0, bytes = 0;
};

struct Layout {
  size_t total = 0;
  Region add(size_t bytes) {
    Region r;
    r.off = (total + 255) & ~size_t(255);
    r.bytes = bytes;
    total = r.off + bytes;
    return r;
  }
};

size_t blk_bytes(int N, int K) { return (size_t)((N + 15) / 16 * 16) * K * 2; }

struct LayerRegions {
  Region ln1, ln2;
  Region dn_in, dn_conv, dn_gnorm, dn_out, S, ring, pend;
  Region at_q, at_k, at_v, at_o, kc, vc, kve;
  Region ffn_gu, ffn_dn;
  Region pf_in, pf_out, pf_qkv, pf_o, pf_gu, pf_dn;   // prefill copies (MkPfW)
};

// The state of sequences 1 .. n_seq - 1 (sequence 0's lives in LayerRegions)
struct SeqLayer {
  Region S, ring, pend, kc, vc, kve;
};
struct SeqRegions {
  Region ctl, layer_table;
  std::vector<SeqLayer> layers;
};

struct Plan {
  int H, V, I, J, nh, dk, dv, C, r_in, nq, nkv, hd, r_in_max, x_o_len, xm_len, max_pages, n_seq;
  Region embed, lnf, rope, page_table, layer_table, ctl, xch, gen;
  std::vector<LayerRegions> layers;
  std::vector<SeqRegions> seq;        // [n_seq - 1]
  // prefill scratch (one pass of MK_PT tokens)
  int K1, NP;
  Region pf_X, pf_a1h, pf_a1l, pf_a2h, pf_a2l, pf_P, pf_cW, pf_cQ, pf_cU, pf_cO, pf_cKt, pf_cg, pf_cd,
      pf_snap, pf_aq, pf_lmbest, pf_part;
  size_t total;
};

int check_config(const mk_config *c, std::string &why) {
  if (!c) { why = "config is NULL"; return MK_EINVAL; }
  if (c->n_layers <= 0 || c->n_layers > 256) { why = "n_layers out of range"; return MK_EINVAL; }
  if (!c->layer_kind) { why = "layer_kind is NULL"; return MK_EINVAL; }
  int nd = 0, na = 0;
  for (int i = 0; i < c->n_layers; ++i) {
    if (c->layer_kind[i] == MK_LAYER_DELTANET) ++nd;
    else if (c->layer_kind[i] == MK_LAYER_ATTENTION) ++na;
    else { why = "layer_kind[" + std::to_string(i) + "] is neither DeltaNet nor attention"; return MK_EINVAL; }
  }
  if (!(c->hidden == 256 || c->hidden == 512 || c->hidden == 1024)) { why = "hidden must be 256, 512 or 1024"; return MK_EINVAL; }
  if (c->vocab <= 0 || c->vocab % 2 != 0) { why = "vocab must be positive and even"; return MK_EINVAL; }
  if (c->ffn <= 0 || c->ffn % 64 != 0) { why = "ffn must be a positive multiple of 64"; return MK_EINVAL; }
  {
    const int J = c->ffn / MK_NX;
    const int G = mk_tile_G(J);
    if (J / 8 / G > 8) { why = "ffn / 8 has too few power-of-two factors for the down-projection tiles"; return MK_EINVAL; }
  }
  if (nd > 0) {
    if (c->dn_heads < 1 || c->dn_heads > MK_NX) { why = "dn_heads must be in [1, 8]"; return MK_EINVAL; }
    if (!(c->dn_dk == 64 || c->dn_dk == 128) || c->dn_dv != c->dn_dk) { why = "dn_dk == dn_dv in {64, 128} required"; return MK_EINVAL; }
    if (c->conv_k != 4) { why = "conv_k must be 4"; return MK_EINVAL; }
  }
  if (na > 0) {
    if (c->at_q_heads < 1 || c->at_q_heads > MK_NX) { why = "at_q_heads must be in [1, 8]"; return MK_EINVAL; }
    if (c->at_kv_heads < 1 || c->at_q_heads % c->at_kv_heads != 0) { why = "at_q_heads must be a multiple of at_kv_heads"; return MK_EINVAL; }
    if (!(c->at_head_dim == 64 || c->at_head_dim == 128)) { why = "at_head_dim must be 64 or 128"; return MK_EINVAL; }
    if (!(c->rope_theta > 0.f)) { why = "rope_theta must be positive"; return MK_EINVAL; }
  }
  if (!(c->rms_eps >= 0.f) || !(c->l2_eps >= 0.f)) { why = "eps must be >= 0"; return MK_EINVAL; }
  if (c->tied_embedding != 1) { why = "only a tied LM head is supported"; return MK_EINVAL; }
  if (c->max_ctx <= 0 || c->max_ctx % MK_PAGE != 0 || c->max_ctx > 10240) { why = "max_ctx must be a multiple of 64 in [64, 10240]"; return MK_EINVAL; }
  if (c->prefill_chunk != 64) { why = "prefill_chunk must be 64"; return MK_EINVAL; }
  if (c->max_verify < 1 || c->max_verify > MK_MAXCOL) { why = "max_verify must be in [1, 5]"; return MK_EINVAL; }
  if (c->kv_quant != 0 && c->kv_quant != 1) { why = "kv_quant must be 0 (bf16 cache) or 1 (8-bit codes)"; return MK_EINVAL; }
  if (c->n_seq < 0 || c->n_seq > MK_MAXCOL) { why = "n_seq must be in [1, 5] (0 means 1)"; return MK_EINVAL; }
  {  // per-wave register budgets of the persistent kernel (weight rows held per phase): each role
     // (token mixer, FFN) has MK_NG workgroups of 8 weight-streaming waves per XCD
    const int Gh = mk_tile_G(c->hidden), RGh = 64 / Gh, XW = MK_NG * MK_WAVES;
    const int J = c->ffn / MK_NX, Gd = mk_tile_G(J);
    if (nd > 0 && c->hidden / (64 / mk_tile_G(c->dn_dv)) > 2 * XW) { why = "DeltaNet out-projection too wide"; return MK_EINVAL; }
    if (na > 0 && c->hidden / (64 / mk_tile_G(c->at_head_dim)) > 2 * XW) { why = "attention o-projection too wide"; return MK_EINVAL; }
    if (nd > 0 && (2 * c->dn_dk + 2 * c->dn_dv + 2) / RGh > 5 * XW) { why = "DeltaNet in-projection too tall"; return MK_EINVAL; }
    if (na > 0 && 3 * c->at_head_dim / RGh > 5 * XW) { why = "QKV projection too tall"; return MK_EINVAL; }
    if (J > 4 * XW) { why = "ffn too large for the gate/up prefetch"; return MK_EINVAL; }
    if (c->hidden / (64 / Gd) > XW) { why = "down-projection tiles too many for one per wave"; return MK_EINVAL; }
  }
  return MK_OK;
}

Plan make_plan(const mk_config *c) {
  Plan p;
  p.H = c->hidden; p.V = c->vocab; p.I = c->ffn; p.J = c->ffn / MK_NX;
  p.nh = c->dn_heads; p.dk = c->dn_dk; p.dv = c->dn_dv;
  p.C = 2 * c->dn_heads * c->dn_dk + c->dn_heads * c->dn_dv;
  p.r_in = 2 * p.dk + 2 * p.dv + 2;
  p.nq = c->at_q_heads; p.nkv = c->at_kv_heads; p.hd = c->at_head_dim;
  bool has_dn = false, has_at = false;
  for (int i = 0; i < c->n_layers; ++i) (c->layer_kind[i] == MK_LAYER_DELTANET ? has_dn : has_at) = true;
  p.r_in_max = std::max(has_dn ? p.r_in : 0, has_at ? 3 * p.hd : 0);
  p.r_in_max = (p.r_in_max + 31) & ~31;  // 256-byte aligned per-column blocks: no cache line is shared

  // DeltaNet: o and o g silu(z) of the head; attention: 16 partials {max, sum, acc[hd]}
  p.x_o_len = std::max(has_dn ? 2 * p.dv : 0, has_at ? MK_NG * (p.hd + 2) : 0);
  p.x_o_len = (p.x_o_len + 31) & ~31;
  p.xm_len = (p.J + 31) & ~31;
  p.max_pages = c->max_ctx / MK_PAGE;
  const size_t H = p.H;
  Layout L;
  p.embed = L.add((size_t)p.V * H * 2);
  p.lnf = L.add(H * 4);
  p.rope = L.add(has_at ? (size_t)c->max_ctx * (p.hd / 2) * 2 * 4 : 0);
  p.page_table = L.add((size_t)p.max_pages * 4);
  p.layer_table = L.add(sizeof(MkLayerDev) * c->n_layers);
  p.ctl = L.add(MK_CTL_WORDS * 4);
  p.layers.resize(c->n_layers);
  for (int i = 0; i < c->n_layers; ++i) {
    LayerRegions &r = p.layers[i];
    r.ln1 = L.add(H * 4);
    r.ln2 = L.add(H * 4);
    if (c->layer_kind[i] == MK_LAYER_DELTANET) {
      r.dn_in = L.add((size_t)p.nh * p.r_in * H * 2);
      r.dn_conv = L.add((size_t)p.C * 4 * 4);
      r.dn_gnorm = L.add((size_t)p.dv * 4);
      r.dn_out = L.add((size_t)p.nh * H * p.dv * 2);
      r.S = L.add((size_t)p.nh * p.dv * p.dk * 4);
      r.ring = L.add((size_t)MK_RING * p.C * 4);
      r.pend = L.add((size_t)2 * p.nh * MK_MAXCOL * mk_pend_stride(p.dv) * 4);
      r.pf_in = L.add(blk_bytes(p.nh * p.r_in, p.H));
      r.pf_out = L.add(blk_bytes(p.H, p.nh * p.dv));
    } else {
      r.pf_qkv = L.add(blk_bytes((p.nq + 2 * p.nkv) * p.hd, p.H));
      r.pf_o = L.add(blk_bytes(p.H, p.nq * p.hd));
      r.at_q = L.add((size_t)p.nq * p.hd * H * 2);
      r.at_k = L.add((size_t)p.nkv * p.hd * H * 2);
      r.at_v = L.add((size_t)p.nkv * p.hd * H * 2);
      r.at_o = L.add((size_t)p.nq * H * p.hd * 2);
      const size_t cb = c->kv_quant ? 1 : 2;   // bytes per cached element: int8 code or bf16
      r.kc = L.add((size_t)p.max_pages * p.nkv * MK_PAGE * p.hd * cb);
      r.vc = L.add((size_t)p.max_pages * p.nkv * MK_PAGE * p.hd * cb);
      r.kve = L.add(c->kv_quant ? (size_t)p.max_pages * p.nkv * MK_PAGE * 2 : 0);
    }
    r.ffn_gu = L.add((size_t)2 * p.I * H * 2);
    r.ffn_dn = L.add((size_t)H * p.I * 2);
    r.pf_gu = L.add(blk_bytes(2 * p.I, p.H));
    r.pf_dn = L.add(blk_bytes(p.H, p.I));
  }
  // sequences 1 .. n_seq - 1: control block, layer table, and per layer the state / KV regions
  p.n_seq = c->n_seq > 0 ? c->n_seq : 1;
  p.seq.resize(p.n_seq - 1);
  for (auto &sq : p.seq) {
    sq.ctl = L.add(MK_CTL_WORDS * 4);
    sq.layer_table = L.add(sizeof(MkLayerDev) * c->n_layers);
    sq.layers.resize(c->n_layers);
    for (int i = 0; i < c->n_layers; ++i) {
      SeqLayer &r = sq.layers[i];
      if (c->layer_kind[i] == MK_LAYER_DELTANET) {
        r.S = L.add((size_t)p.nh * p.dv * p.dk * 4);
        r.ring = L.add((size_t)MK_RING * p.C * 4);
        r.pend = L.add((size_t)2 * p.nh * MK_MAXCOL * mk_pend_stride(p.dv) * 4);
      } else {
        const size_t cb = c->kv_quant ? 1 : 2;
        r.kc = L.add((size_t)p.max_pages * p.nkv * MK_PAGE * p.hd * cb);
        r.vc = L.add((size_t)p.max_pages * p.nkv * MK_PAGE * p.hd * cb);
        r.kve = L.add(c->kv_quant ? (size_t)p.max_pages * p.nkv * MK_PAGE * 2 : 0);
      }
    }
  }
  // exchange slots, sized for the widest launch (verify, MK_MAXCOL columns)
  p.xch = L.add(mk_xch_bytes(MK_MAXCOL, c->n_layers, p.H, p.r_in_max, p.x_o_len, p.xm_len));
  p.gen = L.add(256);   // tokens in, greedy tokens out, n_accepted, error word of mk_generate_lookup
  {
    const size_t T = MK_PT, nch = MK_PT / MK_CHUNK;
    p.K1 = std::max(p.H, std::max(p.nh * p.dv, p.nq * p.hd));
    p.NP = std::max(has_dn ? p.nh * p.r_in : 0, has_at ? (p.nq + 2 * p.nkv) * p.hd : 0);
    p.pf_X = L.add(T * H * 4);
    p.pf_a1h = L.add(T * p.K1 * 2);
    p.pf_a1l = L.add(T * p.K1 * 2);
    p.pf_a2h = L.add(T * p.I * 2);
    p.pf_a2l = L.add(T * p.I * 2);
    p.pf_P = L.add(T * p.NP * 4);
    const size_t nhd = has_dn ? p.nh : 0;
    p.pf_cW = L.add(nhd * nch * MK_CHUNK * p.dk * 4);
    p.pf_cQ = L.add(nhd * nch * MK_CHUNK * p.dk * 4);
    p.pf_cU = L.add(nhd * nch * MK_CHUNK * p.dv * 4);
    p.pf_cO = L.add(nhd * nch * MK_CHUNK * p.dv * 4);
    p.pf_cKt = L.add(nhd * nch * MK_CHUNK * p.dk * 4);
    p.pf_cg = L.add(nhd * nch * MK_CHUNK * 4);
    p.pf_cd = L.add(nhd * nch * MK_CHUNK * 4);
    p.pf_snap = L.add(nhd * nch * p.dv * p.dk * 4);
    p.pf_aq = L.add(has_at ? T * p.nq * p.hd * 4 : 0);
    p.pf_lmbest = L.add((size_t)MK_NWG * 8);
    p.pf_part = L.add((size_t)4 * T * H * 4);
  }
  p.total = (L.total + 255) & ~size_t(255);
  return p;
}

struct Expect {
  std::vector<int64_t> shape;
  const mk_tensor *t = nullptr;
};

std::map<std::string, Expect> expected_tensors(const mk_config *c) {
  std::map<std::string, Expect> e;
  const int64_t H = c->hidden, V = c->vocab, I = c->ffn;
  e["embed"].shape = {V, H};
  e["lnf"].shape = {H};
  for (int i = 0; i < c->n_layers; ++i) {
    const std::string p = "layers." + std::to_string(i) + ".";
    e[p + "ln1"].shape = {H};
    e[p + "ln2"].shape = {H};
    if (c->layer_kind[i] == MK_LAYER_DELTANET) {
      const int64_t qk = (int64_t)c->dn_heads * c->dn_dk, vv = (int64_t)c->dn_heads * c->dn_dv;
      e[p + "dn.wq"].shape = {qk, H};
      e[p + "dn.wk"].shape = {qk, H};
      e[p + "dn.wv"].shape = {vv, H};
      e[p + "dn.wz"].shape = {vv, H};
      e[p + "dn.wa"].shape = {c->dn_heads, H};
      e[p + "dn.wb"].shape = {c->dn_heads, H};
      e[p + "dn.conv"].shape = {2 * qk + vv, c->conv_k};
      e[p + "dn.gnorm"].shape = {c->dn_dv};
      e[p + "dn.wo"].shape = {H, vv};
    } else {
      const int64_t q = (int64_t)c->at_q_heads * c->at_head_dim, kv = (int64_t)c->at_kv_heads * c->at_head_dim;
      e[p + "attn.wq"].shape = {q, H};
      e[p + "attn.wk"].shape = {kv, H};
      e[p + "attn.wv"].shape = {kv, H};
      e[p + "attn.wo"].shape = {H, q};
    }
    e[p + "ffn.wg"].shape = {I, H};
    e[p + "ffn.wu"].shape = {I, H};
    e[p + "ffn.wd"].shape = {H, I};
  }
  return e;
}

// Re-tile rows [rows][K] (row stride src_stride elements) into the tile format of mk_layout.h.
void tile_pack(const uint16_t *src, int rows, int K, size_t src_stride, uint16_t *dst) {
  const int G = mk_tile_G(K), L = K / 8 / G, RG = 64 / G;
  for (int rg = 0; rg < rows / RG; ++rg)
    for (int i = 0; i < L; ++i)
      for (int l = 0; l < 64; ++l) {
        const int row = rg * RG + l / G, chunk = i * G + (l % G);
        std::memcpy(dst + (((size_t)rg * L + i) * 64 + l) * 8, src + (size_t)row * src_stride + (size_t)chunk * 8, 16);
      }
}

// Pack rows [N][K] (row stride src_stride elements) into the GEMM operand block layout of the
// prefill weight copies: 1 KiB blocks of 16 rows x 32 k, block (n / 16, k / 32) at element
// ((n / 16) * (K / 32) + k / 32) * 512; inside a block, row r's 8-element group q sits at 16-byte
// slot 4 r + (q ^ ((r >> 1) & 3)) (the layout in which the GEMM's fragment reads are conflict-free).
// Rows past N are zero.
void blk_pack(const uint16_t *src, int N, int K, size_t src_stride, uint16_t *dst) {
  const int kbn = K / 32, nbn = (N + 15) / 16;
  for (int nb = 0; nb < nbn; ++nb)
    for (int kb = 0; kb < kbn; ++kb)
      for (int r = 0; r < 16; ++r)
        for (int q = 0; q < 4; ++q) {
          const int row = nb * 16 + r, slot = 4 * r + (q ^ ((r >> 1) & 3));
          uint16_t *d = dst + (((size_t)nb * kbn + kb) * 64 + slot) * 8;
          if (row < N) std::memcpy(d, src + (size_t)row * src_stride + (size_t)kb * 32 + q * 8, 16);
          else std::memset(d, 0, 16);
        }
}

inline float bf2f(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

}  // namespace

// ------------------------------------------------------------------------------ ABI
extern "C" const char *mk_status_string(int s) {
  switch (s) {
    case MK_OK: return "ok";
    case MK_EINVAL: return "invalid argument";
    case MK_EDTYPE: return "weight tensor is not BF16";
    case MK_ESHAPE: return "weight tensor missing, duplicated, unknown or mis-shaped";
    case MK_ECTX: return "context length exceeded";
    case MK_ESTATE: return "model not loaded";
    case MK_ELAUNCH: return "device cannot host the persistent grid";
    case MK_EHIP: return "HIP runtime error";
    case MK_EHANG: return "device wait timed out";
    case MK_ETOKEN: return "token id out of range";
    case MK_ENAN: return "non-finite logits";
    default: return "unknown status";
  }
}

extern "C" const char *mk_last_error(void) { return g_err.c_str(); }

extern "C" int mk_required_bytes(const mk_config *cfg, size_t *arena_bytes) {
  std::string why;
  if (!arena_bytes) return fail(MK_EINVAL, "arena_bytes is NULL");
  int s = check_config(cfg, why);
  if (s != MK_OK) return fail(s, why);
  *arena_bytes = make_plan(cfg).total;
  return MK_OK;
}

static int validate_tensors(const mk_config *cfg, const mk_tensor *t, int32_t n,
                            std::map<std::string, Expect> &exp) {
  if (n < 0 || (n > 0 && !t)) return fail(MK_EINVAL, "tensor list is NULL or has a negative length");
  for (int i = 0; i < n; ++i) {
    if (!t[i].name) return fail(MK_EINVAL, "tensor " + std::to_string(i) + " has no name");
    const std::string name = t[i].name;
    auto it = exp.find(name);
    if (it == exp.end()) return fail(MK_ESHAPE, "unknown tensor '" + name + "'");
    if (t[i].dtype != MK_DTYPE_BF16) return fail(MK_EDTYPE, "tensor '" + name + "' is not BF16");
    if (it->second.t) return fail(MK_ESHAPE, "tensor '" + name + "' given twice");
    const auto &sh = it->second.shape;
    bool ok = t[i].ndim == (int32_t)sh.size();
    for (size_t d = 0; ok && d < sh.size(); ++d) ok = t[i].shape[d] == sh[d];
    if (!ok) return fail(MK_ESHAPE, "tensor '" + name + "' has the wrong shape");
    if (!t[i].data) return fail(MK_EINVAL, "tensor '" + name + "' has no data");
    if (t[i].on_device != 0 && t[i].on_device != 1) return fail(MK_EINVAL, "tensor '" + name + "': on_device must be 0 or 1");
    it->second.t = &t[i];
  }
  for (auto &kv : exp)
    if (!kv.second.t) return fail(MK_ESHAPE, "tensor '" + kv.first + "' is missing");
  (void)cfg;
  return MK_OK;
}

static int check_device(int *dev) {
  HIPCHECK(hipGetDevice(dev));
  hipDeviceProp_t prop;
  HIPCHECK(hipGetDeviceProperties(&prop, *dev));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(MK_ELAUNCH, std::string("device is ") + prop.gcnArchName + ", need gfx950 (MI355X)");
  if (prop.multiProcessorCount != MK_NWG)
    return fail(MK_ELAUNCH, "device has " + std::to_string(prop.multiProcessorCount) + " CUs, need 256 (8 XCDs x 32)");
  for (int variant = 0; variant < MK_N_VARIANTS + 2; ++variant)
    for (int tmpl : {1, MK_MAXCOL}) {
      // (variants past MK_N_VARIANTS: the batch instantiations, MK_MAXCOL columns only)
      const int v = variant < MK_N_VARIANTS ? variant : MK_BATCH | (variant - MK_N_VARIANTS);
      if (v >= MK_N_VARIANTS && tmpl == 1) continue;
      int per_cu = 0;
      HIPCHECK(mk_forward_occupancy(tmpl, v, &per_cu));
      if (per_cu < 1) return fail(MK_ELAUNCH, "persistent kernel does not fit on a CU");
    }
  return MK_OK;
}

extern "C" int mk_load_weights(const mk_config *cfg, const mk_tensor *tensors, int32_t n_tensors, void *d_arena,
                               size_t arena_bytes, void *stream, mk_model **out) {
  std::string why;
  if (!out) return fail(MK_EINVAL, "out is NULL");
  *out = nullptr;
  int s = check_config(cfg, why);
  if (s != MK_OK) return fail(s, why);
  auto exp = expected_tensors(cfg);
  s = validate_tensors(cfg, tensors, n_tensors, exp);
  if (s != MK_OK) return s;
  Plan p = make_plan(cfg);
  if (!d_arena) return fail(MK_EINVAL, "arena is NULL");
  if (((uintptr_t)d_arena & 255) != 0) return fail(MK_EINVAL, "arena is not 256-byte aligned");
  if (arena_bytes < p.total) return fail(MK_EINVAL, "arena too small: need " + std::to_string(p.total) + " bytes");

  int dev = 0;
  s = check_device(&dev);
  if (s != MK_OK) return s;
  void *static_xch = nullptr;   // the static exchange slots of this device (looked up once per device)
  HIPCHECK(mk_static_scratch(&static_xch));
  hipStream_t st = (hipStream_t)stream;
  char *A = (char *)d_arena;
  // tensors in device memory: host copies for the re-tiling below
  std::map<std::string, std::vector<uint16_t>> host_copy;
  HIPCHECK(hipStreamSynchronize(st));
  for (auto &kv : exp) {
    const mk_tensor *t = kv.second.t;
    if (!t->on_device) continue;
    size_t n = 1;
    for (int64_t d : kv.second.shape) n *= (size_t)d;
    std::vector<uint16_t> &h = host_copy[kv.first];
    h.resize(n);
    HIPCHECK(hipMemcpy(h.data(), t->data, n * 2, hipMemcpyDeviceToHost));
  }
  auto T = [&](const std::string &name) {
    auto it = host_copy.find(name);
    return it != host_copy.end() ? (const uint16_t *)it->second.data() : (const uint16_t *)exp[name].t->data;
  };
  auto put = [&](const Region &r, const void *host) -> hipError_t {
    hipError_t e = hipMemcpyAsync(A + r.off, host, r.bytes, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return e;
    return hipStreamSynchronize(st);  // the staging buffer is reused right after
  };
  auto gains = [&](const uint16_t *src, size_t n) {
    std::vector<float> g(n);
    for (size_t i = 0; i < n; ++i) g[i] = bf2f(src[i]);
    return g;
  };
  const size_t H = p.H;
  std::vector<uint16_t> stage;
  // embedding / LM head: tile format with one row group per G-lane segment == row-major for H <= 1024
  HIPCHECK(put(p.embed, T("embed")));
  { auto g = gains(T("lnf"), H); HIPCHECK(put(p.lnf, g.data())); }

  MkDev d{};
  d.n_layers = cfg->n_layers; d.H = p.H; d.V = p.V; d.I = p.I; d.J = p.J;
  d.nh = p.nh; d.dk = p.dk; d.dv = p.dv; d.C = p.C; d.r_in = p.r_in;
  d.nq = p.nq; d.nkv = p.nkv; d.hd = p.hd; d.r_in_max = p.r_in_max; d.x_o_len = p.x_o_len; d.xm_len = p.xm_len;
  d.max_ctx = cfg->max_ctx; d.max_pages = p.max_pages;
  d.kv_quant = cfg->kv_quant;
  d.rms_eps = cfg->rms_eps; d.l2_eps = cfg->l2_eps;
  d.embed = (const uint16_t *)(A + p.embed.off);
  d.lnf = (const float *)(A + p.lnf.off);
  d.rope = (const float *)(A + p.rope.off);
  d.page_table = (const int32_t *)(A + p.page_table.off);
  d.layers = (const MkLayerDev *)(A + p.layer_table.off);
  d.ctl = (int32_t *)(A + p.ctl.off);

  if (p.rope.bytes) {  // rotary table in double precision, stored as float
    std::vector<float> rt((size_t)cfg->max_ctx * (p.hd / 2) * 2);
    for (int pos = 0; pos < cfg->max_ctx; ++pos)
      for (int i = 0; i < p.hd / 2; ++i) {
        const double invf = std::pow((double)cfg->rope_theta, -2.0 * i / (double)p.hd);
        const double ang = (double)pos * invf;
        rt[((size_t)pos * (p.hd / 2) + i) * 2 + 0] = (float)std::cos(ang);
        rt[((size_t)pos * (p.hd / 2) + i) * 2 + 1] = (float)std::sin(ang);
      }
    HIPCHECK(put(p.rope, rt.data()));
  }
  {
    std::vector<int32_t> pt(p.max_pages);
    for (int i = 0; i < p.max_pages; ++i) pt[i] = i;  // one sequence: identity page map
    HIPCHECK(put(p.page_table, pt.data()));
  }

  std::vector<MkLayerDev> lt(cfg->n_layers);
  std::vector<MkPfW> pfw(cfg->n_layers);
  std::vector<std::pair<size_t, size_t>> state;
  // a prefill weight copy: rows [N][K] packed into the GEMM block layout and uploaded
  auto put_blk = [&](const Region &r, const uint16_t *src, int N, int K, size_t src_stride) -> hipError_t {
    stage.assign(r.bytes / 2, 0);
    blk_pack(src, N, K, src_stride, stage.data());
    return put(r, stage.data());
  };
  int nd = 0, na = 0;
  for (int li = 0; li < cfg->n_layers; ++li) {
    const LayerRegions &r = p.layers[li];
    MkLayerDev &L = lt[li];
    std::memset(&L, 0, sizeof(L));
    const std::string pre = "layers." + std::to_string(li) + ".";
    L.kind = cfg->layer_kind[li] == MK_LAYER_DELTANET ? 0 : 1;
    L.idx = L.kind == 0 ? nd++ : na++;
    { auto g = gains(T(pre + "ln1"), H); HIPCHECK(put(r.ln1, g.data())); }
    { auto g = gains(T(pre + "ln2"), H); HIPCHECK(put(r.ln2, g.data())); }
    L.ln1 = (const float *)(A + r.ln1.off);
    L.ln2 = (const float *)(A + r.ln2.off);
    if (L.kind == 0) {
      const int nh = p.nh, dk = p.dk, dv = p.dv;
      stage.assign(r.dn_in.bytes / 2, 0);
      std::vector<uint16_t> rows((size_t)p.r_in * H), all((size_t)nh * p.r_in * H);
      for (int h = 0; h < nh; ++h) {
        size_t o = 0;
        auto take = [&](const uint16_t *src, int r0, int nr) {
          std::memcpy(rows.data() + o * H, src + (size_t)r0 * H, (size_t)nr * H * 2);
          o += nr;
        };
        take(T(pre + "dn.wq"), h * dk, dk);
        take(T(pre + "dn.wk"), h * dk, dk);
        take(T(pre + "dn.wv"), h * dv, dv);
        take(T(pre + "dn.wz"), h * dv, dv);
        take(T(pre + "dn.wa"), h, 1);
        take(T(pre + "dn.wb"), h, 1);
        tile_pack(rows.data(), p.r_in, p.H, H, stage.data() + (size_t)h * p.r_in * H);
        std::memcpy(all.data() + (size_t)h * p.r_in * H, rows.data(), rows.size() * 2);
      }
      HIPCHECK(put(r.dn_in, stage.data()));
      HIPCHECK(put_blk(r.pf_in, all.data(), nh * p.r_in, p.H, H));
      HIPCHECK(put_blk(r.pf_out, T(pre + "dn.wo"), p.H, nh * dv, (size_t)nh * dv));
      pfw[li].in = (const uint16_t *)(A + r.pf_in.off);
      pfw[li].out = (const uint16_t *)(A + r.pf_out.off);
      { auto g = gains(T(pre + "dn.conv"), (size_t)p.C * 4); HIPCHECK(put(r.dn_conv, g.data())); }
      { auto g = gains(T(pre + "dn.gnorm"), dv); HIPCHECK(put(r.dn_gnorm, g.data())); }
      stage.assign(r.dn_out.bytes / 2, 0);
      for (int h = 0; h < nh; ++h)
        tile_pack(T(pre + "dn.wo") + (size_t)h * dv, p.H, dv, (size_t)nh * dv, stage.data() + (size_t)h * H * dv);
      HIPCHECK(put(r.dn_out, stage.data()));
      L.dn_in = (const uint16_t *)(A + r.dn_in.off);
      L.dn_conv = (const float *)(A + r.dn_conv.off);
      L.dn_gnorm = (const float *)(A + r.dn_gnorm.off);
      L.dn_out = (const uint16_t *)(A + r.dn_out.off);
      L.S = (float *)(A + r.S.off);
      L.ring = (float *)(A + r.ring.off);
      L.pend = (float *)(A + r.pend.off);
      state.push_back({r.S.off, r.S.bytes});
      state.push_back({r.ring.off, r.ring.bytes});
      state.push_back({r.pend.off, r.pend.bytes});
    } else {
      const int nq = p.nq, nkv = p.nkv, hd = p.hd;
      stage.assign(r.at_q.bytes / 2, 0);
      for (int i = 0; i < nq; ++i) tile_pack(T(pre + "attn.wq") + (size_t)i * hd * H, hd, p.H, H, stage.data() + (size_t)i * hd * H);
      HIPCHECK(put(r.at_q, stage.data()));
      stage.assign(r.at_k.bytes / 2, 0);
      for (int i = 0; i < nkv; ++i) tile_pack(T(pre + "attn.wk") + (size_t)i * hd * H, hd, p.H, H, stage.data() + (size_t)i * hd * H);
      HIPCHECK(put(r.at_k, stage.data()));
      stage.assign(r.at_v.bytes / 2, 0);
      for (int i = 0; i < nkv; ++i) tile_pack(T(pre + "attn.wv") + (size_t)i * hd * H, hd, p.H, H, stage.data() + (size_t)i * hd * H);
      HIPCHECK(put(r.at_v, stage.data()));
      stage.assign(r.at_o.bytes / 2, 0);
      for (int i = 0; i < nq; ++i) tile_pack(T(pre + "attn.wo") + (size_t)i * hd, p.H, hd, (size_t)nq * hd, stage.data() + (size_t)i * H * hd);
      HIPCHECK(put(r.at_o, stage.data()));
      {
        std::vector<uint16_t> qkv((size_t)(nq + 2 * nkv) * hd * H);
        std::memcpy(qkv.data(), T(pre + "attn.wq"), (size_t)nq * hd * H * 2);
        std::memcpy(qkv.data() + (size_t)nq * hd * H, T(pre + "attn.wk"), (size_t)nkv * hd * H * 2);
        std::memcpy(qkv.data() + (size_t)(nq + nkv) * hd * H, T(pre + "attn.wv"), (size_t)nkv * hd * H * 2);
        HIPCHECK(put_blk(r.pf_qkv, qkv.data(), (nq + 2 * nkv) * hd, p.H, H));
      }
      HIPCHECK(put_blk(r.pf_o, T(pre + "attn.wo"), p.H, nq * hd, (size_t)nq * hd));
      pfw[li].qkv = (const uint16_t *)(A + r.pf_qkv.off);
      pfw[li].o = (const uint16_t *)(A + r.pf_o.off);
      L.at_q = (const uint16_t *)(A + r.at_q.off);
      L.at_k = (const uint16_t *)(A + r.at_k.off);
      L.at_v = (const uint16_t *)(A + r.at_v.off);
      L.at_o = (const uint16_t *)(A + r.at_o.off);
      L.kc = A + r.kc.off;
      L.vc = A + r.vc.off;
      L.kve = cfg->kv_quant ? (int8_t *)(A + r.kve.off) : nullptr;
    }
    {
      const int J = p.J;
      stage.assign(r.ffn_gu.bytes / 2, 0);
      std::vector<uint16_t> rows((size_t)2 * J * H);
      for (int xg = 0; xg < MK_NX; ++xg) {
        for (int j = 0; j < J; ++j) {
          std::memcpy(rows.data() + (size_t)(2 * j) * H, T(pre + "ffn.wg") + (size_t)(xg * J + j) * H, H * 2);
          std::memcpy(rows.data() + (size_t)(2 * j + 1) * H, T(pre + "ffn.wu") + (size_t)(xg * J + j) * H, H * 2);
        }
        tile_pack(rows.data(), 2 * J, p.H, H, stage.data() + (size_t)xg * 2 * J * H);
      }
      HIPCHECK(put(r.ffn_gu, stage.data()));
      stage.assign(r.ffn_dn.bytes / 2, 0);
      for (int xg = 0; xg < MK_NX; ++xg)
        tile_pack(T(pre + "ffn.wd") + (size_t)xg * J, p.H, J, (size_t)p.I, stage.data() + (size_t)xg * H * J);
      HIPCHECK(put(r.ffn_dn, stage.data()));
      {
        std::vector<uint16_t> gu((size_t)2 * p.I * H);
        for (int i = 0; i < p.I; ++i) {
          std::memcpy(gu.data() + (size_t)(2 * i) * H, T(pre + "ffn.wg") + (size_t)i * H, H * 2);
          std::memcpy(gu.data() + (size_t)(2 * i + 1) * H, T(pre + "ffn.wu") + (size_t)i * H, H * 2);
        }
        HIPCHECK(put_blk(r.pf_gu, gu.data(), 2 * p.I, p.H, H));
      }
      HIPCHECK(put_blk(r.pf_dn, T(pre + "ffn.wd"), p.H, p.I, (size_t)p.I));
      pfw[li].gu = (const uint16_t *)(A + r.pf_gu.off);
      pfw[li].dn = (const uint16_t *)(A + r.pf_dn.off);
      L.ffn_gu = (const uint16_t *)(A + r.ffn_gu.off);
      L.ffn_dn = (const uint16_t *)(A + r.ffn_dn.off);
    }
  }
  HIPCHECK(put(p.layer_table, lt.data()));
  // the other sequences: the same weights, their own state and KV cache
  std::vector<MkDev> seq_dev(p.n_seq, d);
  std::vector<std::vector<MkLayerDev>> seq_lt(p.n_seq, lt);
  for (int sq = 1; sq < p.n_seq; ++sq) {
    const SeqRegions &R = p.seq[sq - 1];
    for (int li = 0; li < cfg->n_layers; ++li) {
      MkLayerDev &L = seq_lt[sq][li];
      const SeqLayer &r = R.layers[li];
      if (L.kind == 0) {
        L.S = (float *)(A + r.S.off);
        L.ring = (float *)(A + r.ring.off);
        L.pend = (float *)(A + r.pend.off);
        state.push_back({r.S.off, r.S.bytes});
        state.push_back({r.ring.off, r.ring.bytes});
        state.push_back({r.pend.off, r.pend.bytes});
      } else {
        L.kc = A + r.kc.off;
        L.vc = A + r.vc.off;
        L.kve = cfg->kv_quant ? (int8_t *)(A + r.kve.off) : nullptr;
      }
    }
    HIPCHECK(put(R.layer_table, seq_lt[sq].data()));
    seq_dev[sq].layers = (const MkLayerDev *)(A + R.layer_table.off);
    seq_dev[sq].ctl = (int32_t *)(A + R.ctl.off);
    state.push_back({R.ctl.off, R.ctl.bytes});
  }
  // exchange slots start with tag 0 (never used); control words and state start at zero
  {
    const size_t x0 = p.xch.off;
    HIPCHECK(hipMemsetAsync(A + x0, 0, p.total - x0, st));
  }
  state.push_back({p.ctl.off, p.ctl.bytes});
  for (auto &r : state) HIPCHECK(hipMemsetAsync(A + r.first, 0, r.second, st));
  HIPCHECK(hipStreamSynchronize(st));

  mk_model *mm = new mk_model();
  mm->magic = MK_MAGIC;
  mm->device = dev;
  mm->cfg = *cfg;
  mm->kinds.assign(cfg->layer_kind, cfg->layer_kind + cfg->n_layers);
  mm->cfg.layer_kind = mm->kinds.data();
  mm->dev = d;
  mm->layers_host = lt;
  mm->pfw = pfw;
  mm->cur = 0;
  mm->seq_dev = seq_dev;
  mm->seq_layers_host = seq_lt;
  mm->seq_pos_hi.assign(p.n_seq, 0);
  mm->seq_verified.assign(p.n_seq, 0);
  {
    MkPf &f = mm->pf;
    auto P = [&](const Region &r) { return (void *)(A + r.off); };
    f.X = (float *)P(p.pf_X);
    f.a1h = (uint16_t *)P(p.pf_a1h); f.a1l = (uint16_t *)P(p.pf_a1l);
    f.a2h = (uint16_t *)P(p.pf_a2h); f.a2l = (uint16_t *)P(p.pf_a2l);
    f.P = (float *)P(p.pf_P);
    f.cW = (float *)P(p.pf_cW); f.cQ = (float *)P(p.pf_cQ); f.cU = (float *)P(p.pf_cU); f.cO = (float *)P(p.pf_cO);
    f.cKt = (float *)P(p.pf_cKt); f.cg = (float *)P(p.pf_cg); f.cd = (float *)P(p.pf_cd);
    f.snap = (float *)P(p.pf_snap);
    f.aq = (float *)P(p.pf_aq);
    f.lmbest = (unsigned long long *)P(p.pf_lmbest);
    f.part = (float *)P(p.pf_part);
    f.K1 = p.K1; f.NP = p.NP;
  }
  mm->arena = A;
  mm->arena_bytes = arena_bytes;
  mm->xch = (uint2 *)(A + p.xch.off);
  mm->gen = (int32_t *)(A + p.gen.off);
  mm->static_xch = (uint2 *)static_xch;
  mm->state_regions = state;
  mm->pos_hi = 0;
  mm->tag = 1;
  *out = mm;
  return MK_OK;
}

static bool live(const mk_model *m) { return m && m->magic == MK_MAGIC; }

extern "C" int mk_reset_state(mk_model *m, void *stream) {
  if (!live(m)) return fail(MK_ESTATE, "model not loaded");
  hipStream_t st = (hipStream_t)stream;
  for (auto &r : m->state_regions) HIPCHECK(hipMemsetAsync(m->arena + r.first, 0, r.second, st));
  m->pos_hi = 0;
  m->seq_pos_hi.assign(m->seq_pos_hi.size(), 0);
  m->seq_verified.assign(m->seq_verified.size(), 0);
  return MK_OK;
}

static int sync_pos(mk_model *m, hipStream_t st, int32_t *ctl_out) {
  int32_t ctl[MK_CTL_WORDS];
  HIPCHECK(hipStreamSynchronize(st));
  HIPCHECK(hipMemcpy(ctl, m->dev.ctl, sizeof(ctl), hipMemcpyDeviceToHost));
  m->pos_hi = ctl[MK_CTL_POS];
  if (ctl_out) std::memcpy(ctl_out, ctl, sizeof(ctl));
  return MK_OK;
}

static int ensure_ctx(mk_model *m, int32_t n, hipStream_t st) {
  if ((int64_t)m->pos_hi + n <= m->cfg.max_ctx) return MK_OK;
  int s = sync_pos(m, st, nullptr);  // the bound is loose after a verify: read the real position
  if (s != MK_OK) return s;
  if ((int64_t)m->pos_hi + n > m->cfg.max_ctx)
    return fail(MK_ECTX, "position " + std::to_string(m->pos_hi) + " + " + std::to_string(n) + " tokens exceeds max_ctx");
  return MK_OK;
}

extern "C" int mk_prefill(mk_model *m, const int32_t *d_tokens, int32_t n_tokens, int32_t *d_next_token,
                          float *d_last_logits, void *stream) {
  if (!live(m)) return fail(MK_ESTATE, "model not loaded");
  if (!d_tokens || !d_next_token) return fail(MK_EINVAL, "token buffers must not be NULL");
  if (n_tokens < 1 || n_tokens > m->cfg.max_ctx) return fail(MK_EINVAL, "n_tokens out of range");
  hipStream_t st = (hipStream_t)stream;
  int s = ensure_ctx(m, n_tokens, st);
  if (s != MK_OK) return s;
  if (m->pf_blocks >= 2 && !m->pf_side) {
    int cur = 0;
    HIPCHECK(hipGetDevice(&cur));
    HIPCHECK(hipSetDevice(m->device));
    hipError_t e = hipStreamCreateWithFlags(&m->pf_side, hipStreamNonBlocking);
    for (int i = 0; e == hipSuccess && i < m->dev.n_layers + 2; ++i) {
      hipEvent_t ev;
      e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
      if (e == hipSuccess) m->pf_ev.push_back(ev);
    }
    (void)hipSetDevice(cur);
    HIPCHECK(e);
  }
  const bool two = m->pf_blocks >= 2 && m->pf_side;
  HIPCHECK(mk_prefill_enqueue(&m->dev, m->layers_host.data(), &m->pf, d_tokens, n_tokens, d_next_token, d_last_logits, st,
                              two ? m->pf_side : nullptr, two ? m->pf_ev.data() : nullptr, m->pf_blocks,
                              m->pfw.data()));
  m->pos_hi += n_tokens;
  m->seq_verified[m->cur] = 0;   // the prefill applies any pending updates first
  return MK_OK;
}

// Sequence numbers of the static exchange slots, one counter per device: every launch that uses
// them tags its slots with a number no earlier launch on the device used.
static std::mutex g_static_mu;
static uint32_t g_static_tag[256];

static int decode_launch(mk_model *m, const int32_t *d_tokens, int32_t n_tokens, int32_t *d_argmax, float *d_logits,
                         int32_t *d_n_accepted, void *stream, bool use_static) {
  if (!live(m)) return fail(MK_ESTATE, "model not loaded");
  if (!d_tokens || !d_argmax) return fail(MK_EINVAL, "token buffers must not be NULL");
  if (n_tokens < 1 || n_tokens > m->cfg.max_verify) return fail(MK_EINVAL, "n_tokens must be in [1, max_verify]");
  const int tmpl = n_tokens == 1 ? 1 : MK_MAXCOL;
  if (use_static) {
    const size_t need = mk_xch_bytes(tmpl, m->dev.n_layers, m->dev.H, m->dev.r_in_max, m->dev.x_o_len, m->dev.xm_len);
    if (need > (size_t)MK_STATIC_SCRATCH_BYTES)
      return fail(MK_EINVAL, "the exchange slots of this launch need " + std::to_string(need) +
                                 " bytes, more than the static array's " + std::to_string((size_t)MK_STATIC_SCRATCH_BYTES));
    if (m->device < 0 || m->device >= 256) return fail(MK_EINVAL, "device index out of range");
  }
  hipStream_t st = (hipStream_t)stream;
  int s = ensure_ctx(m, n_tokens, st);
  if (s != MK_OK) return s;
  MkLaunch a{};
  a.m = m->dev;
  a.tokens = d_tokens;
  a.n = n_tokens;
  a.argmax = d_argmax;
  a.logits = d_logits;
  a.n_acc = d_n_accepted;
  if (use_static) {
    std::lock_guard<std::mutex> lock(g_static_mu);
    uint32_t &t = g_static_tag[m->device];
    if (++t == 0) t = 1;                   // 0 is the tag of never-written slots
    a.tag0 = t;
    a.xch = m->static_xch;
  } else {
    a.tag0 = m->tag;
    a.xch = m->xch;
  }
  HIPCHECK(mk_launch_forward(&a, tmpl, mk_variant_of(m->dev), st));
  if (!use_static) m->tag += 1;
  m->pos_hi += n_tokens;
  m->seq_verified[m->cur] = n_tokens > 1;
  return MK_OK;
}

extern "C" int mk_decode_step(mk_model *m, const int32_t *d_tokens, int32_t n_tokens, int32_t *d_argmax,
                              float *d_logits, int32_t *d_n_accepted, void *stream) {
  return decode_launch(m, d_tokens, n_tokens, d_argmax, d_logits, d_n_accepted, stream, false);
}

extern "C" int mk_decode_step_static(mk_model *m, const int32_t *d_tokens, int32_t n_tokens, int32_t *d_argmax,
                                     float *d_logits, int32_t *d_n_accepted, void *stream) {
  return decode_launch(m, d_tokens, n_tokens, d_argmax, d_logits, d_n_accepted, stream, true);
}

extern "C" int mk_sync_status(mk_model *m, void *stream, int32_t *pos) {
  if (!live(m)) return fail(MK_ESTATE, "model not loaded");
  int32_t ctl[MK_CTL_WORDS];
  int s = sync_pos(m, (hipStream_t)stream, ctl);
  if (s != MK_OK) return s;
  if (pos) *pos = ctl[MK_CTL_POS];
  // device errors of a batch launch land in the control block of its first column's sequence:
  // report the first sequence with one (the selected sequence first)
  for (size_t q = 0; q < m->seq_dev.size() && ctl[MK_CTL_ERR] == 0; ++q) {
    if ((int)q == m->cur) continue;
    int32_t other[MK_CTL_WORDS];
    HIPCHECK(hipMemcpy(other, m->seq_dev[q].ctl, sizeof(other), hipMemcpyDeviceToHost));
    if (other[MK_CTL_ERR] != 0) {
      for (int w = MK_CTL_ERR; w < MK_CTL_WHERE + 4; ++w) ctl[w] = other[w];
    }
  }
  const int e = ctl[MK_CTL_ERR];
  if (e & MK_DERR_XCD) return fail(MK_ELAUNCH, "workgroups were not placed round-robin over the XCDs from one starting XCD");
  if (e & MK_DERR_HANG) {
    char buf[160];
    std::snprintf(buf, sizeof(buf), "a device-side wait timed out (step %d layer %d phase %d, block %d thread %d, tag seen %u wanted %u)",
                  (ctl[MK_CTL_WHERE] >> 16) & 16383, (ctl[MK_CTL_WHERE] >> 8) & 255, ctl[MK_CTL_WHERE] & 255,
                  ctl[MK_CTL_WHERE + 1] >> 16, ctl[MK_CTL_WHERE + 1] & 65535, (unsigned)ctl[MK_CTL_WHERE + 2],
                  (unsigned)ctl[MK_CTL_WHERE + 3]);
    return fail(MK_EHANG, buf);
  }
  if (e & MK_DERR_TOKEN) return fail(MK_ETOKEN, "a token id was out of range");
  if (e & MK_DERR_NAN) return fail(MK_ENAN, "non-finite logits");
  return MK_OK;
}

// ------------------------------------------------------------------------------ sequences
extern "C" int mk_select_seq(mk_model *m, int32_t seq) {
  if (!live(m)) return fail(MK_ESTATE, "model not loaded");
  if (seq < 0 || seq >= (int32_t)m->seq_dev.size())
    return fail(MK_EINVAL, "seq " + std::to_string(seq) + " out of range [0, " + std::to_string(m->seq_dev.size()) + ")");
  m->seq_pos_hi[m->cur] = m->pos_hi;
  m->cur = seq;
  m->dev = m->seq_dev[seq];
  m->layers_host = m->seq_layers_host[seq];
  m->pos_hi = m->seq_pos_hi[seq];
  return MK_OK;
}

extern "C" int mk_decode_batch(mk_model *m, const int32_t *seqs, int32_t n, const int32_t *d_tokens, int32_t *d_argmax,
                               float *d_logits, void *stream) {
  if (!live(m)) return fail(MK_ESTATE, "model not loaded");
  if (!seqs || !d_tokens || !d_argmax) return fail(MK_EINVAL, "seqs and token buffers must not be NULL");
  const int nseq = (int)m->seq_dev.size();
  if (n < 1 || n > nseq) return fail(MK_EINVAL, "n must be in [1, n_seq]");
  if (m->cfg.kv_quant) return fail(MK_EINVAL, "batch decode needs the bf16 KV cache (kv_quant = 0)");
  m->seq_pos_hi[m->cur] = m->pos_hi;
  hipStream_t st = (hipStream_t)stream;
  for (int32_t c = 0; c < n; ++c) {
    const int q = seqs[c];
    if (q < 0 || q >= nseq) return fail(MK_EINVAL, "seqs[" + std::to_string(c) + "] out of range");
    for (int32_t j = 0; j < c; ++j)
      if (seqs[j] == q) return fail(MK_EINVAL, "seqs must be distinct");
    if (m->seq_verified[q])
      return fail(MK_EINVAL, "sequence " + std::to_string(q) +
                                 " last ran a verify forward: a decode step or prefill on it must settle it first");
    if ((int64_t)m->seq_pos_hi[q] + 1 > m->cfg.max_ctx) {
      int32_t ctl[MK_CTL_WORDS];
      HIPCHECK(hipStreamSynchronize(st));
      HIPCHECK(hipMemcpy(ctl, m->seq_dev[q].ctl, sizeof(ctl), hipMemcpyDeviceToHost));
      m->seq_pos_hi[q] = ctl[MK_CTL_POS];
      if ((int64_t)m->seq_pos_hi[q] + 1 > m->cfg.max_ctx)
        return fail(MK_ECTX, "sequence " + std::to_string(q) + " is at max_ctx");
    }
  }
  MkLaunch a{};
  a.m = m->seq_dev[seqs[0]];
  a.tokens = d_tokens;
  a.n = n;
  a.argmax = d_argmax;
  a.logits = d_logits;
  a.n_acc = nullptr;
  for (int32_t c = 0; c < n; ++c) {
    a.seq_layers[c] = m->seq_dev[seqs[c]].layers;
    a.seq_ctl[c] = m->seq_dev[seqs[c]].ctl;
  }
  a.tag0 = m->tag;
  a.xch = m->xch;
  // a batch of one is a decode step of that sequence: the one-column kernel (same arithmetic)
  if (n == 1) HIPCHECK(mk_launch_forward(&a, 1, mk_variant_of(a.m), st));
  else HIPCHECK(mk_launch_forward(&a, MK_MAXCOL, mk_shape_of(m->dev) | MK_BATCH, st));
  m->tag += 1;
  for (int32_t c = 0; c < n; ++c) m->seq_pos_hi[seqs[c]] += 1;
  m->pos_hi = m->seq_pos_hi[m->cur];
  return MK_OK;
}

// ------------------------------------------------------------------------------ lookup drafts
extern "C" int mk_lookup_draft(const int32_t *history, int32_t n_history, int32_t ngram_min, int32_t ngram_max,
                               int32_t max_draft, int32_t *out_draft) {
  if (n_history < 0 || max_draft < 0 || ngram_min < 1 || ngram_max < ngram_min)
    return fail(MK_EINVAL, "mk_lookup_draft: need n_history >= 0, max_draft >= 0, 1 <= ngram_min <= ngram_max");
  if (max_draft == 0 || n_history < 2) return 0;
  if (!history || !out_draft) return fail(MK_EINVAL, "mk_lookup_draft: NULL buffer");
  for (int32_t g = std::min(ngram_max, n_history - 1); g >= ngram_min; --g) {
    const int32_t *suf = history + (n_history - g);
    // most recent earlier occurrence: start i with i + g < n_history (at least one token follows it)
    for (int32_t i = n_history - g - 1; i >= 0; --i) {
      if (std::memcmp(history + i, suf, (size_t)g * sizeof(int32_t)) != 0) continue;
      const int32_t nd = std::min(max_draft, n_history - (i + g));
      std::memcpy(out_draft, history + i + g, (size_t)nd * sizeof(int32_t));
      return nd;
    }
  }
  return 0;
}

extern "C" int mk_generate_lookup(mk_model *m, const int32_t *history, int32_t n_history, int32_t last_token,
                                  int32_t n_generate, int32_t ngram_min, int32_t ngram_max, int32_t *out_tokens,
                                  mk_lookup_stats *stats, void *stream) {
  if (!live(m)) return fail(MK_ESTATE, "model not loaded");
  if (n_history < 0 || (n_history > 0 && !history)) return fail(MK_EINVAL, "history must hold n_history tokens");
  if (n_generate < 0 || (n_generate > 0 && !out_tokens)) return fail(MK_EINVAL, "out_tokens must hold n_generate tokens");
  if (ngram_min < 1 || ngram_max < ngram_min) return fail(MK_EINVAL, "need 1 <= ngram_min <= ngram_max");
  if (last_token < 0 || last_token >= m->cfg.vocab) return fail(MK_EINVAL, "last_token out of range");
  mk_lookup_stats st{0, 0, 0};
  if (stats) *stats = st;
  hipStream_t s = (hipStream_t)stream;
  std::vector<int32_t> ctx(history, history + n_history);
  ctx.push_back(last_token);
  int32_t *d_tok = m->gen, *d_arg = m->gen + 16, *d_nacc = m->gen + 32;
  int32_t cur = last_token, done = 0;
  int32_t tok[MK_MAXCOL], arg[MK_MAXCOL], draft[MK_MAXCOL];
  while (done < n_generate) {
    const int32_t rem = n_generate - done;
    const int32_t dmax = std::min(m->cfg.max_verify - 1, rem - 1);
    int32_t nd = dmax > 0 ? mk_lookup_draft(ctx.data(), (int32_t)ctx.size(), ngram_min, ngram_max, dmax, draft) : 0;
    if (nd < 0) return nd;
    tok[0] = cur;
    for (int32_t i = 0; i < nd; ++i) tok[1 + i] = draft[i];
    HIPCHECK(hipMemcpyAsync(d_tok, tok, (size_t)(1 + nd) * sizeof(int32_t), hipMemcpyHostToDevice, s));
    int r = decode_launch(m, d_tok, 1 + nd, d_arg, nullptr, nd > 0 ? d_nacc : nullptr, stream, false);
    if (r != MK_OK) return r;
    int32_t nacc = 1, ctl[MK_CTL_WORDS];
    HIPCHECK(hipMemcpyAsync(arg, d_arg, (size_t)(1 + nd) * sizeof(int32_t), hipMemcpyDeviceToHost, s));
    if (nd > 0) HIPCHECK(hipMemcpyAsync(&nacc, d_nacc, sizeof(int32_t), hipMemcpyDeviceToHost, s));
    HIPCHECK(hipMemcpyAsync(ctl, m->dev.ctl, sizeof(ctl), hipMemcpyDeviceToHost, s));
    HIPCHECK(hipStreamSynchronize(s));
    m->pos_hi = ctl[MK_CTL_POS];
    if (ctl[MK_CTL_ERR] != 0) return mk_sync_status(m, stream, nullptr);   // reports the device error
    if (nacc < 1 || nacc > 1 + nd) return fail(MK_EHIP, "n_accepted out of range");
    for (int32_t i = 0; i < nacc; ++i) {
      out_tokens[done + i] = arg[i];
      ctx.push_back(arg[i]);
    }
    done += nacc;
    cur = arg[nacc - 1];
    st.forwards += 1;
    st.drafted += nd;
    st.accepted += nacc - 1;
    if (stats) *stats = st;
  }
  return MK_OK;
}

extern "C" int mk_set_prefill_blocks(mk_model *m, int32_t max_blocks) {
  if (!live(m)) return fail(MK_ESTATE, "model not loaded");
  if (max_blocks != 1 && max_blocks != 2) return fail(MK_EINVAL, "max_blocks must be 1 or 2");
  m->pf_blocks = max_blocks;
  return MK_OK;
}

extern "C" void mk_free(mk_model *m) {
  if (!live(m)) return;
  m->magic = 0;
  if (m->pf_side) {   // its work is ordered before later work on the caller's stream; let it drain
    (void)hipStreamSynchronize(m->pf_side);
    for (hipEvent_t e : m->pf_ev) (void)hipEventDestroy(e);
    (void)hipStreamDestroy(m->pf_side);
  }
  delete m;
}
