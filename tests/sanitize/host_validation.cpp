// Host-side argument validation of every C ABI entry point, run against a build of the library
// whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer, whose objects hold no
// device code, and which is linked with a stand-in for the HIP runtime that has no device
// (tests/sanitize/hip_stub.cpp), so nothing here can run on a GPU.  Each case calls one entry point and
// compares its status with the one the header documents; a call whose arguments are valid gets
// as far as its launch, which the stand-in checks and fails (OSCAR_ERR_HIP).  Any sanitizer report
// aborts the process.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "oscar.h"

namespace {

int g_failed = 0, g_run = 0;

void expect(const char* what, long long got, long long want) {
  ++g_run;
  if (got != want) {
    ++g_failed;
    std::fprintf(stderr, "FAIL %s: got %lld, want %lld\n", what, got, want);
  }
}

constexpr int32_t OK = OSCAR_OK, INV = OSCAR_ERR_INVALID_ARGUMENT, UNS = OSCAR_ERR_UNSUPPORTED,
                  SMALL = OSCAR_ERR_WORKSPACE_TOO_SMALL, HIP = OSCAR_ERR_HIP;

// Stand-ins for device buffers: aligned, never dereferenced on the host (the library only
// checks them and hands them to launches, which fail without a device).
alignas(256) unsigned char g_buf[4096];
void* const A = g_buf;
void* const MIS = g_buf + 4;   // 4-byte aligned, not 16-byte aligned
void* const MIS2 = g_buf + 2;  // 2-byte aligned

template <class T>
T* p(void* v) { return static_cast<T*>(v); }

oscar_layout layout(int sink = 4, int window = 128) {
  oscar_layout l;
  l.num_kv_heads = 8;
  l.head_dim = 128;
  l.page_size = 16;
  l.group_size = 32;
  l.num_sink = sink;
  l.window = window;
  l.num_pages = 1024;
  l.max_pages_per_seq = 64;
  l.num_slots = 64;
  return l;
}

const size_t kBig = (size_t)1 << 40;   // "large enough" workspace size for validation

// ---- appends ------------------------------------------------------------------------------

struct AppendArgs {
  const oscar_layout* lay;
  void *pages, *sinkwin, *bt, *k, *v, *off, *start, *rk, *rv, *mean;
  int32_t batch, total;
  float ck, cv;
  int32_t method;
};

AppendArgs append_args(const oscar_layout* lay) {
  return AppendArgs{lay, A, A, A, A, A, A, A, A, A, nullptr, 4, 64, 1.0f, 0.9f, OSCAR_APPEND_AUTO};
}

int32_t call_append_ex(const AppendArgs& a) {
  return oscar_rotate_quantize_append_ex(a.lay, p<uint8_t>(a.pages), p<uint16_t>(a.sinkwin),
                                         p<int32_t>(a.bt), nullptr, a.batch, a.total,
                                         p<uint16_t>(a.k), p<uint16_t>(a.v), p<int32_t>(a.off),
                                         p<int32_t>(a.start), p<float>(a.rk), p<float>(a.rv),
                                         p<float>(a.mean), a.ck, a.cv, a.method, nullptr);
}
int32_t call_append(const AppendArgs& a) {
  return oscar_rotate_quantize_append(a.lay, p<uint8_t>(a.pages), p<uint16_t>(a.sinkwin),
                                      p<int32_t>(a.bt), nullptr, a.batch, a.total,
                                      p<uint16_t>(a.k), p<uint16_t>(a.v), p<int32_t>(a.off),
                                      p<int32_t>(a.start), p<float>(a.rk), p<float>(a.rv), a.ck,
                                      a.cv, nullptr);
}
int32_t call_hadamard(const AppendArgs& a) {
  return oscar_rotate_quantize_append_hadamard(
      a.lay, p<uint8_t>(a.pages), p<uint16_t>(a.sinkwin), p<int32_t>(a.bt), nullptr, a.batch,
      a.total, p<uint16_t>(a.k), p<uint16_t>(a.v), p<int32_t>(a.off), p<int32_t>(a.start),
      p<int8_t>(a.rk), p<int8_t>(a.rv), a.ck, a.cv, nullptr);
}
int32_t call_int4_append(const AppendArgs& a) {
  return oscar_int4_rotate_quantize_append(a.lay, p<uint8_t>(a.pages), p<uint16_t>(a.sinkwin),
                                           p<int32_t>(a.bt), nullptr, a.batch, a.total,
                                           p<uint16_t>(a.k), p<uint16_t>(a.v), p<int32_t>(a.off),
                                           p<int32_t>(a.start), p<float>(a.rk), p<float>(a.rv),
                                           p<float>(a.mean), a.ck, a.cv, nullptr);
}
int32_t call_bf16_append(const AppendArgs& a) {
  return oscar_bf16_append(a.lay, p<uint16_t>(a.pages), p<int32_t>(a.bt), a.batch, a.total,
                           p<uint16_t>(a.k), p<uint16_t>(a.v), p<int32_t>(a.off),
                           p<int32_t>(a.start), nullptr);
}

void layout_cases() {
  // Every layout field, through the prepared decode (the cheapest caller of check_layout).
  auto dec = [](const oscar_layout* l) {
    return oscar_decode_attention_prepared(l, p<uint8_t>(A), p<uint16_t>(A), p<int32_t>(A),
                                           nullptr, 1, 32, p<int32_t>(A), 0.088f, 0, 4, A, kBig,
                                           nullptr);
  };
  expect("layout null", dec(nullptr), INV);
  struct Case { const char* what; void (*edit)(oscar_layout&); int32_t want; };
  const Case cases[] = {
      {"head_dim 256", [](oscar_layout& l) { l.head_dim = 256; }, UNS},
      {"head_dim 0", [](oscar_layout& l) { l.head_dim = 0; }, UNS},
      {"page_size 8", [](oscar_layout& l) { l.page_size = 8; }, UNS},
      {"group_size 16", [](oscar_layout& l) { l.group_size = 16; }, UNS},
      {"hkv 0", [](oscar_layout& l) { l.num_kv_heads = 0; }, INV},
      {"hkv 65536", [](oscar_layout& l) { l.num_kv_heads = 65536; }, INV},
      {"hkv INT_MIN", [](oscar_layout& l) { l.num_kv_heads = INT_MIN; }, INV},
      {"sink -1", [](oscar_layout& l) { l.num_sink = -1; }, INV},
      {"window INT_MIN", [](oscar_layout& l) { l.window = INT_MIN; }, INV},
      {"sink+window INT_MAX+INT_MAX", [](oscar_layout& l) { l.num_sink = INT_MAX; l.window = INT_MAX; }, UNS},
      {"sink INT_MAX", [](oscar_layout& l) { l.num_sink = INT_MAX; l.window = 1; }, UNS},
      {"sink+window 257", [](oscar_layout& l) { l.num_sink = 129; l.window = 128; }, UNS},
      {"pages -1", [](oscar_layout& l) { l.num_pages = -1; }, INV},
      {"max_pages 0", [](oscar_layout& l) { l.max_pages_per_seq = 0; }, INV},
      {"max_pages INT_MIN", [](oscar_layout& l) { l.max_pages_per_seq = INT_MIN; }, INV},
      {"slots -1", [](oscar_layout& l) { l.num_slots = -1; }, INV},
  };
  for (const Case& c : cases) {
    oscar_layout l = layout();
    c.edit(l);
    expect(c.what, dec(&l), c.want);
  }
  oscar_layout full = layout(128, 128);   // S + W = 256, the largest supported
  expect("sink+window 256 reaches the launch", dec(&full), HIP);
  oscar_layout none = layout(0, 0);
  expect("no sink/window store needed", oscar_decode_attention_prepared(
             &none, p<uint8_t>(A), nullptr, p<int32_t>(A), nullptr, 1, 32, p<int32_t>(A), 0.088f,
             0, 4, A, kBig, nullptr), HIP);
}

void append_cases() {
  const oscar_layout lay = layout();
  using Fn = int32_t (*)(const AppendArgs&);
  const struct { const char* name; Fn fn; bool has_clip, has_rot, has_mean; } calls[] = {
      {"append", call_append, true, true, false},
      {"append_ex", call_append_ex, true, true, true},
      {"hadamard", call_hadamard, true, false, false},
      {"int4_append", call_int4_append, true, true, true},
      {"bf16_append", call_bf16_append, false, false, false},
  };
  char what[128];
  for (const auto& c : calls) {
    auto run = [&](const char* tag, AppendArgs a, int32_t want) {
      std::snprintf(what, sizeof what, "%s: %s", c.name, tag);
      expect(what, c.fn(a), want);
    };
    AppendArgs a = append_args(&lay);
    run("valid decode-token append", a, HIP);
    AppendArgs b = a; b.total = 300; run("valid 300 rows", b, HIP);
    b = a; b.total = 1 << 30; run("2^30 rows", b, HIP);
    b = a; b.total = (1 << 30) + 1; run("2^30 + 1 rows", b, UNS);
    b = a; b.total = INT_MAX; run("INT_MAX rows", b, UNS);
    b = a; b.total = INT_MIN; run("INT_MIN rows", b, INV);
    b = a; b.batch = -1; run("batch -1", b, INV);
    b = a; b.batch = 0; run("batch 0", b, OK);
    b = a; b.total = 0; run("no rows", b, OK);
    b = a; b.lay = nullptr; run("layout null", b, INV);
    b = a; b.pages = nullptr; run("pages null", b, INV);
    b = a; b.bt = nullptr; run("block table null", b, INV);
    b = a; b.k = nullptr; run("k null", b, INV);
    b = a; b.v = nullptr; run("v null", b, INV);
    b = a; b.off = nullptr; run("offsets null", b, INV);
    b = a; b.start = nullptr; run("start null", b, INV);
    b = a; b.pages = MIS; run("pages misaligned", b, INV);
    b = a; b.k = MIS; run("k misaligned", b, INV);
    b = a; b.v = MIS; run("v misaligned", b, INV);
    if (c.fn != call_bf16_append) {
      b = a; b.sinkwin = nullptr; run("store null with sink/window rows", b, INV);
      b = a; b.sinkwin = MIS; run("store misaligned", b, INV);
    }
    if (c.has_clip) {
      const float bad[] = {0.0f, -0.5f, 1.5f, NAN, INFINITY};
      for (float x : bad) {
        b = a; b.ck = x; run("clip_k outside (0, 1]", b, INV);
        b = a; b.cv = x; run("clip_v outside (0, 1]", b, INV);
      }
    }
    if (c.has_rot) {
      b = a; b.rk = nullptr; run("rot_k null", b, INV);
      b = a; b.rv = MIS; run("rot_v misaligned", b, INV);
    }
    if (c.has_mean) {
      b = a; b.mean = A; run("key mean", b, HIP);
      b = a; b.mean = MIS2; run("key mean misaligned", b, INV);
    }
  }
  oscar_layout none = layout(0, 0);
  AppendArgs a = append_args(&none);
  a.sinkwin = nullptr;
  expect("append: no store needed without sink/window rows", call_append(a), HIP);
  a = append_args(&lay);
  for (int32_t m : {-1, 3, INT_MAX}) {
    AppendArgs b = a;
    b.method = m;
    expect("append_ex: unknown method", call_append_ex(b), INV);
  }
  for (int32_t m : {OSCAR_APPEND_VECTOR, OSCAR_APPEND_MATRIX}) {
    AppendArgs b = a;
    b.method = m;
    b.total = 2000;
    expect("append_ex: explicit method", call_append_ex(b), HIP);
  }
}

// ---- decode family ------------------------------------------------------------------------

struct DecodeArgs {
  const oscar_layout* lay;
  void *pages, *sinkwin, *bt, *q, *lens, *rk, *rv, *ws, *out;
  int32_t batch, hq, nw, ms;
  float sm;
  size_t wsb;
};

DecodeArgs decode_args(const oscar_layout* lay) {
  return DecodeArgs{lay, A, A, A, A, A, A, A, A, A, 1, 32, 0, 4, 0.088f, kBig};
}

int32_t call_decode(const DecodeArgs& a) {
  return oscar_decode_attention(a.lay, p<uint8_t>(a.pages), p<uint16_t>(a.sinkwin),
                                p<int32_t>(a.bt), nullptr, a.batch, a.hq, p<uint16_t>(a.q),
                                p<int32_t>(a.lens), p<float>(a.rk), a.sm, a.nw, a.ms, a.ws, a.wsb,
                                nullptr);
}
int32_t call_prepare(const DecodeArgs& a) {
  return oscar_prepare_queries(a.lay, a.batch, a.hq, p<uint16_t>(a.q), p<int32_t>(a.lens),
                               p<float>(a.rk), a.nw, a.ms, a.ws, a.wsb, nullptr);
}
int32_t call_prepared(const DecodeArgs& a) {
  return oscar_decode_attention_prepared(a.lay, p<uint8_t>(a.pages), p<uint16_t>(a.sinkwin),
                                         p<int32_t>(a.bt), nullptr, a.batch, a.hq,
                                         p<int32_t>(a.lens), a.sm, a.nw, a.ms, a.ws, a.wsb,
                                         nullptr);
}
int32_t call_static(const DecodeArgs& a) {
  return oscar_decode_attention_static(a.lay, p<uint8_t>(a.pages), p<uint16_t>(a.sinkwin),
                                       p<int32_t>(a.bt), nullptr, a.batch, a.hq,
                                       p<uint16_t>(a.q), p<int32_t>(a.lens), p<float>(a.rk),
                                       p<float>(a.rv), a.sm, a.nw, a.ms, p<float>(a.out),
                                       nullptr, nullptr);
}
// INT4 and BF16 decode take split_pages in place of num_workers (nw + 16 here, so >= 1).
int32_t call_int4(const DecodeArgs& a) {
  return oscar_int4_decode_attention(a.lay, p<uint8_t>(a.pages), p<uint16_t>(a.sinkwin),
                                     p<int32_t>(a.bt), nullptr, a.batch, a.hq, p<uint16_t>(a.q),
                                     p<int32_t>(a.lens), p<float>(a.rk), a.sm, a.nw + 16, a.ms,
                                     a.ws, a.wsb, nullptr);
}
int32_t call_bf16(const DecodeArgs& a) {
  return oscar_bf16_decode_attention(a.lay, p<uint16_t>(a.pages), p<int32_t>(a.bt), a.batch,
                                     a.hq, p<uint16_t>(a.q), p<int32_t>(a.lens), a.sm, a.nw + 16,
                                     a.ms, a.ws, a.wsb, nullptr);
}

void decode_cases() {
  const oscar_layout lay = layout();
  using Fn = int32_t (*)(const DecodeArgs&);
  const struct { const char* name; Fn fn; bool workers, workspace, static_ws; } calls[] = {
      {"decode", call_decode, true, true, false},
      {"prepare", call_prepare, true, true, false},
      {"prepared", call_prepared, true, true, false},
      {"static", call_static, true, false, true},
      {"int4_decode", call_int4, false, true, false},
      {"bf16_decode", call_bf16, false, true, false},
  };
  char what[128];
  for (const auto& c : calls) {
    auto run = [&](const char* tag, DecodeArgs a, int32_t want) {
      std::snprintf(what, sizeof what, "%s: %s", c.name, tag);
      expect(what, c.fn(a), want);
    };
    const DecodeArgs a = decode_args(&lay);
    DecodeArgs b = a;
    run("valid batch 1", a, HIP);
    b = a; b.batch = 64; run("valid batch 64", b, HIP);
    b = a; b.batch = 0; run("batch 0", b, OK);
    b = a; b.batch = -1; run("batch -1", b, INV);
    b = a; b.batch = INT_MIN; run("batch INT_MIN", b, INV);
    b = a; b.hq = 30; run("hq not a multiple of hkv", b, INV);
    b = a; b.hq = 24; run("group 3", b, UNS);
    b = a; b.hq = 128; run("group 16", b, UNS);
    b = a; b.hq = 0; run("hq 0", b, INV);
    b = a; b.hq = INT_MIN; run("hq INT_MIN", b, INV);
    b = a; b.ms = 0; run("max_splits 0", b, INV);
    b = a; b.ms = 65536; run("max_splits 65536", b, INV);
    b = a; b.ms = INT_MAX; run("max_splits INT_MAX", b, INV);
    b = a; b.ms = 2000; run("max_splits beyond the combine's LDS", b, UNS);
    b = a; b.hq = 64; b.ms = 760; run("G 8 at the LDS limit", b, HIP);
    b = a; b.hq = 64; b.ms = 761; run("G 8 beyond the LDS limit", b, UNS);
    if (c.workers) {
      b = a; b.nw = -1; run("num_workers -1", b, INV);
      b = a; b.nw = (1 << 20) + 1; run("num_workers 2^20 + 1", b, INV);
      b = a; b.nw = 1 << 20; run("num_workers 2^20", b, HIP);
    }
    // 2^22 sequences x 32 heads = 2^27 rows: accepted; one more sequence is not
    {
      oscar_layout l1 = layout();
      l1.max_pages_per_seq = 1;
      b = a; b.lay = &l1; b.batch = 1 << 22;
      run("2^27 query rows", b, c.static_ws ? SMALL : HIP);
      b.batch = (1 << 22) + 1;
      run("2^27 + 32 query rows", b, UNS);
      b.batch = INT_MAX;
      // the INT2 plan check (batch * hkv * max_pages < 2^31) comes first where it exists
      run("batch INT_MAX", b, UNS);
    }
    if (c.fn != call_prepare) {
      const float bad[] = {NAN, INFINITY, -INFINITY, 0.0f, -0.0f, -0.088f};
      for (float x : bad) { b = a; b.sm = x; run("bad softmax scale", b, INV); }
      b = a; b.pages = nullptr; run("pages null", b, INV);
      b = a; b.pages = MIS; run("pages misaligned", b, INV);
      b = a; b.bt = nullptr; run("block table null", b, INV);
      if (c.fn != call_bf16) {
        b = a; b.sinkwin = nullptr; run("store null with sink/window rows", b, INV);
        b = a; b.sinkwin = MIS; run("store misaligned", b, INV);
      }
    }
    if (c.fn != call_prepared) {
      b = a; b.q = nullptr; run("q null", b, INV);
      b = a; b.q = MIS; run("q misaligned", b, INV);
      if (c.fn != call_bf16) {
        b = a; b.rk = nullptr; run("rot_k null", b, INV);
        b = a; b.rk = MIS; run("rot_k misaligned", b, INV);
      }
    }
    b = a; b.lens = nullptr; run("seq_lens null", b, INV);
    if (c.workspace) {
      b = a; b.ws = nullptr; run("workspace null", b, INV);
      b = a; b.ws = MIS; run("workspace misaligned", b, INV);
      b = a; b.wsb = 100; run("workspace too small", b, SMALL);
      b = a; b.wsb = oscar_decode_workspace_bytes(a.batch, a.hq, a.ms);
      run("workspace exactly the size", b, HIP);
      b.wsb -= 1;
      run("workspace one byte short", b, SMALL);
    }
    if (c.static_ws) {
      b = a; b.out = nullptr; run("out null", b, INV);
      b = a; b.rv = MIS; run("rot_v misaligned", b, INV);
      b = a; b.rv = nullptr; run("no rot_v", b, HIP);
      b = a; b.batch = 64; b.ms = 8; run("within the static workspace", b, HIP);
    }
  }
}

void append_prepare_cases() {
  const oscar_layout lay = layout();
  auto call = [&](int32_t batch, int32_t total, int32_t hq, void* pages, void* k, void* km,
                  float ck, void* q, void* ws, size_t wsb, int32_t nw, int32_t ms) {
    return oscar_append_and_prepare(&lay, p<uint8_t>(pages), p<uint16_t>(A), p<int32_t>(A),
                                    nullptr, batch, total, p<uint16_t>(k), p<uint16_t>(A),
                                    p<int32_t>(A), p<int32_t>(A), p<float>(A), p<float>(A),
                                    p<float>(km), ck, 0.9f, hq, p<uint16_t>(q), p<int32_t>(A), nw,
                                    ms, ws, wsb, nullptr);
  };
  expect("append_prepare: valid, one launch", call(64, 64, 32, A, A, nullptr, 1.0f, A, A, kBig, 0, 4), HIP);
  expect("append_prepare: valid, 255 rows", call(64, 255, 32, A, A, nullptr, 1.0f, A, A, kBig, 0, 4), HIP);
  expect("append_prepare: valid, two launches", call(64, 256, 32, A, A, nullptr, 1.0f, A, A, kBig, 0, 4), HIP);
  expect("append_prepare: valid, key mean", call(4, 4, 32, A, A, A, 1.0f, A, A, kBig, 0, 4), HIP);
  expect("append_prepare: no new rows", call(4, 0, 32, nullptr, nullptr, nullptr, 1.0f, A, A, kBig, 0, 4), HIP);
  expect("append_prepare: G 8", call(4, 4, 64, A, A, nullptr, 1.0f, A, A, kBig, 0, 4), HIP);
  expect("append_prepare: 2^27 rows", call(1 << 22, 64, 32, A, A, nullptr, 1.0f, A, A, kBig, 0, 4), UNS);
  expect("append_prepare: batch 0", call(0, 64, 32, A, A, nullptr, 1.0f, A, A, kBig, 0, 4), OK);
  expect("append_prepare: batch -1", call(-1, 64, 32, A, A, nullptr, 1.0f, A, A, kBig, 0, 4), INV);
  expect("append_prepare: total -1", call(4, -1, 32, A, A, nullptr, 1.0f, A, A, kBig, 0, 4), INV);
  expect("append_prepare: total INT_MAX", call(4, INT_MAX, 32, A, A, nullptr, 1.0f, A, A, kBig, 0, 4), UNS);
  expect("append_prepare: hq 30", call(4, 4, 30, A, A, nullptr, 1.0f, A, A, kBig, 0, 4), INV);
  expect("append_prepare: hq 24", call(4, 4, 24, A, A, nullptr, 1.0f, A, A, kBig, 0, 4), UNS);
  expect("append_prepare: clip 0", call(4, 4, 32, A, A, nullptr, 0.0f, A, A, kBig, 0, 4), INV);
  expect("append_prepare: clip NaN", call(4, 4, 32, A, A, nullptr, NAN, A, A, kBig, 0, 4), INV);
  expect("append_prepare: pages null", call(4, 4, 32, nullptr, A, nullptr, 1.0f, A, A, kBig, 0, 4), INV);
  expect("append_prepare: k misaligned", call(4, 4, 32, A, MIS, nullptr, 1.0f, A, A, kBig, 0, 4), INV);
  expect("append_prepare: key mean misaligned", call(4, 4, 32, A, A, MIS2, 1.0f, A, A, kBig, 0, 4), INV);
  expect("append_prepare: q null", call(4, 4, 32, A, A, nullptr, 1.0f, nullptr, A, kBig, 0, 4), INV);
  expect("append_prepare: workspace small", call(4, 4, 32, A, A, nullptr, 1.0f, A, A, 100, 0, 4), SMALL);
  expect("append_prepare: workspace misaligned", call(4, 4, 32, A, A, nullptr, 1.0f, A, MIS, kBig, 0, 4), INV);
  expect("append_prepare: workers -1", call(4, 4, 32, A, A, nullptr, 1.0f, A, A, kBig, -1, 4), INV);
  expect("append_prepare: max_splits 65536", call(4, 4, 32, A, A, nullptr, 1.0f, A, A, kBig, 0, 65536), INV);
}

void combine_cases() {
  auto comb = [](int32_t batch, int32_t hq, int32_t hkv, int32_t ms, void* ws, size_t wsb,
                 void* rv, void* out) {
    return oscar_combine(batch, hq, hkv, ms, ws, wsb, p<float>(rv), p<float>(out), nullptr,
                         nullptr);
  };
  expect("combine: valid", comb(1, 32, 8, 4, A, kBig, A, A), HIP);
  expect("combine: no rot_v", comb(1, 32, 8, 4, A, kBig, nullptr, A), HIP);
  expect("combine: small workspace", comb(1, 32, 8, 4, A, 100, A, A), SMALL);
  expect("combine: workspace null", comb(1, 32, 8, 4, nullptr, kBig, A, A), INV);
  expect("combine: workspace misaligned", comb(1, 32, 8, 4, MIS, kBig, A, A), INV);
  expect("combine: out null", comb(1, 32, 8, 4, A, kBig, A, nullptr), INV);
  expect("combine: rot_v misaligned", comb(1, 32, 8, 4, A, kBig, MIS, A), INV);
  expect("combine: hq 33", comb(1, 33, 8, 4, A, kBig, A, A), INV);
  expect("combine: hkv 0", comb(1, 32, 0, 4, A, kBig, A, A), INV);
  expect("combine: hkv INT_MIN", comb(1, 32, INT_MIN, 4, A, kBig, A, A), INV);
  expect("combine: max_splits 65536", comb(1, 32, 8, 65536, A, kBig, A, A), INV);
  expect("combine: batch -1", comb(-1, 32, 8, 4, A, kBig, A, A), INV);
  expect("combine: batch 0", comb(0, 32, 8, 4, A, kBig, A, A), OK);
  expect("combine: 2^27 rows", comb(1 << 22, 32, 8, 4, A, kBig, A, A), HIP);
  expect("combine: more than 2^27 rows", comb(1 << 23, 32, 8, 4, A, kBig, A, A), UNS);
  expect("combine: batch INT_MAX", comb(INT_MAX, 32, 8, 4, A, (size_t)-1, A, A), UNS);
}

void workspace_cases() {
  expect("ws: batch -1", (long long)oscar_decode_workspace_bytes(-1, 32, 4), 0);
  expect("ws: hq 0", (long long)oscar_decode_workspace_bytes(1, 0, 4), 0);
  expect("ws: max_splits 0", (long long)oscar_decode_workspace_bytes(1, 32, 0), 0);
  expect("ws: max_splits 65536", (long long)oscar_decode_workspace_bytes(1, 32, 65536), 0);
  expect("ws: max_splits INT_MAX", (long long)oscar_decode_workspace_bytes(1, 32, INT_MAX), 0);
  expect("ws: batch INT_MAX", (long long)oscar_decode_workspace_bytes(INT_MAX, 32, 4), 0);
  expect("ws: hq INT_MAX", (long long)oscar_decode_workspace_bytes(1, INT_MAX, 4), 0);
  expect("ws: batch 0", (long long)oscar_decode_workspace_bytes(0, 32, 4), 256);
  // the documented formula, at a small and at the largest accepted size
  const struct { int32_t b, hq, ms; } sizes[] = {{1, 32, 4}, {64, 32, 64}, {3, 8, 1},
                                                  {1 << 22, 32, 65535}, {1 << 27, 1, 65535}};
  for (const auto& s : sizes) {
    const unsigned long long rows = (unsigned long long)s.b * s.hq;
    const unsigned long long plan = (4ULL * (4 + 3ULL * s.b + rows) + 255) / 256 * 256;
    const unsigned long long want = rows * (1024 + ((unsigned long long)s.ms + 8) * 520) + plan;
    expect("ws: formula", (long long)oscar_decode_workspace_bytes(s.b, s.hq, s.ms), (long long)want);
  }
}

void probe_cases() {
  auto rr = [](void* pool, int32_t nrec, void* ids, int32_t n, int32_t nw, void* out) {
    return oscar_read_records(p<uint8_t>(pool), nrec, p<int32_t>(ids), n, nw, p<uint32_t>(out),
                              nullptr);
  };
  expect("read_records: valid", rr(A, 8, A, 8, 4, A), HIP);
  expect("read_records: n INT_MAX", rr(A, 8, A, INT_MAX, 1 << 20, A), HIP);
  expect("read_records: n -1", rr(A, 8, A, -1, 4, A), INV);
  expect("read_records: no records", rr(A, 0, A, 8, 4, A), INV);
  expect("read_records: no workers", rr(A, 8, A, 8, 0, A), INV);
  expect("read_records: 2^20 + 1 workers", rr(A, 8, A, 8, (1 << 20) + 1, A), INV);
  expect("read_records: pool null", rr(nullptr, 8, A, 8, 4, A), INV);
  expect("read_records: ids null", rr(A, 8, nullptr, 8, 4, A), INV);
  expect("read_records: out null", rr(A, 8, A, 8, 4, nullptr), INV);
  expect("read_records: pool misaligned", rr(MIS, 8, A, 8, 4, A), INV);
  expect("read_records: n 0", rr(nullptr, 8, nullptr, 0, 4, nullptr), OK);

  auto mf = [](void* a, void* b, void* c, void* d, int32_t tiles) {
    return oscar_mfma_bf16_tiles(p<uint16_t>(a), p<uint16_t>(b), p<float>(c), p<float>(d), tiles,
                                 nullptr);
  };
  expect("mfma tiles: valid", mf(A, A, A, A, 4), HIP);
  expect("mfma tiles: 2^20", mf(A, A, A, A, 1 << 20), HIP);
  expect("mfma tiles: 2^20 + 1", mf(A, A, A, A, (1 << 20) + 1), INV);
  expect("mfma tiles: -1", mf(A, A, A, A, -1), INV);
  expect("mfma tiles: 0", mf(nullptr, nullptr, nullptr, nullptr, 0), OK);
  expect("mfma tiles: a null", mf(nullptr, A, A, A, 4), INV);
  expect("mfma tiles: d null", mf(A, A, A, nullptr, 4), INV);
}

void status_cases() {
  const struct { int32_t code; const char* text; } known[] = {
      {OK, "ok"}, {INV, "invalid argument"}, {UNS, "unsupported geometry"},
      {SMALL, "workspace too small"}, {HIP, "HIP launch failure"}};
  for (const auto& k : known) expect(k.text, std::strcmp(oscar_status_string(k.code), k.text), 0);
  for (int32_t code : {-1, 5, INT_MAX, INT_MIN})
    expect("unknown status", std::strcmp(oscar_status_string(code), "unknown status"), 0);
}

}  // namespace

// Launch counters of the HIP stand-in the sanitized library is linked with.
extern "C" long oscar_stub_launches();
extern "C" long oscar_stub_bad_launches();

int main() {
  layout_cases();
  append_cases();
  decode_cases();
  append_prepare_cases();
  combine_cases();
  workspace_cases();
  probe_cases();
  status_cases();
  // valid calls got as far as their launches, and every launch shape the host code computed
  // (at the limits too) was a legal one
  expect("launches attempted", oscar_stub_launches() >= 50, 1);
  expect("launches with an invalid shape", oscar_stub_bad_launches(), 0);
  std::printf("host validation: %d cases, %ld launches, %d failed\n", g_run,
              oscar_stub_launches(), g_failed);
  return g_failed == 0 ? 0 : 1;
}
