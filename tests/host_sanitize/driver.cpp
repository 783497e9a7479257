// Drives every entry point of the C ABI (include/tq.h) through its argument
// checks and, with the host stand-ins of fake_runtime.cpp, through its
// successful paths, for shapes on the single-kernel and the general path.
// Built with -fsanitize=address,undefined: any out-of-bounds access, use
// after free, leak or undefined operation in the host code fails the run.
// Exit status 0 and a final "ok" line when every expected status matched.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/tq.h"

extern int g_launches;

static int g_checks = 0, g_fail = 0;
#define EXPECT(call, want)                                                                     \
  do {                                                                                         \
    const long long got_ = (long long)(call);                                                  \
    ++g_checks;                                                                                \
    if (got_ != (long long)(want)) {                                                           \
      ++g_fail;                                                                                \
      std::fprintf(stderr, "%s:%d: %s = %lld, expected %lld (%s)\n", __FILE__, __LINE__, #call, \
                   got_, (long long)(want), tq_last_error());                                  \
    }                                                                                          \
  } while (0)
#define EXPECT_TRUE(cond) EXPECT((cond) ? 1 : 0, 1)

// "Device" buffers: host memory of exactly the requested size (so that ASan
// reports an access one byte past it), 256-byte aligned, released at the
// end of the scope.
struct Buf {
  void* p = nullptr;
  size_t n = 0;
  explicit Buf(size_t bytes) : n(bytes) {
    if (bytes && posix_memalign(&p, 256, bytes) == 0) std::memset(p, 0, bytes);
  }
  ~Buf() { std::free(p); }
  Buf(const Buf&) = delete;
  Buf& operator=(const Buf&) = delete;
  template <class T> T* as() const { return (T*)p; }
};

static uint16_t half_bits(float f) {
  _Float16 h = (_Float16)f;
  uint16_t b;
  std::memcpy(&b, &h, 2);
  return b;
}

static void size_queries() {
  tq_config ok{128, 64, 3, 3};
  EXPECT(tq_config_key_record_bytes(&ok), 64);
  EXPECT(tq_value_block_bytes(&ok), 4 * (4 * 3 * 128 + 128));
  EXPECT(tq_cache_key_bytes(&ok, 3, 256), 3 * 256 * 64);
  EXPECT(tq_cache_key_bytes(&ok, 3, 100), 0);
  tq_config half{64, 32, 2, 4};
  EXPECT(tq_config_key_record_bytes(&half), 4 * (2 * 64 / 32 + 1 + 2));
  const tq_config bad[] = {{100, 64, 3, 3}, {128, 48, 3, 3}, {128, 64, -1, 3}, {128, 64, 3, 5},
                           {128, 64, 3, 0}, {2048, 64, 3, 3}, {96, 64, 3, 3}, {32, 32, 3, 3},
                           {1088, 64, 3, 3}, {128, 576, 3, 3}};
  for (const tq_config& c : bad) {
    EXPECT(tq_config_key_record_bytes(&c), 0);
    EXPECT(tq_workspace_bytes(&c, 1, 4, 100), 0);
    EXPECT(tq_topk_workspace_bytes(&c, 1, 4, 100, 10), 0);
    std::vector<double> R((size_t)std::max(c.head_dim, 1) * std::max(c.head_dim, 1), 0.0);
    std::vector<double> S((size_t)std::max(c.proj_dim, 1) * std::max(c.head_dim, 1), 1.0);
    tq_ctx* h = nullptr;
    EXPECT(tq_create(&c, R.data(), S.data(), &h), TQ_EINVAL);
    EXPECT_TRUE(h == nullptr);
  }
  EXPECT(tq_config_key_record_bytes(nullptr), 0);
  EXPECT(tq_workspace_bytes(&ok, 1, 513, 100), 0);
  EXPECT(tq_workspace_bytes(&ok, 0, 4, 100), 0);
  EXPECT(tq_topk_workspace_bytes(&ok, 1, 4, 100, 17), 0);
  EXPECT(tq_key_record_bytes(nullptr), 0);
  EXPECT(tq_value_record_bytes(nullptr), 0);
  EXPECT(tq_attend_workspace_bytes(nullptr, 1, 4, 100), 0);
  EXPECT(tq_append_workspace_bytes(nullptr, 1, 100), 0);
}

static void codebooks() {
  for (int d : {1, 64, 128, 1024})
    for (int b = 0; b <= 4; ++b) {
      std::vector<double> c(16, 0.0), beta(16, 0.0);
      EXPECT(tq_lloyd_max_codebook(d, b, c.data(), b ? beta.data() : nullptr), TQ_OK);
      for (int i = 1; i < (1 << b); ++i) EXPECT_TRUE(c[i] > c[i - 1]);
    }
  double c[16], beta[16];
  EXPECT(tq_lloyd_max_codebook(0, 3, c, beta), TQ_EINVAL);
  EXPECT(tq_lloyd_max_codebook(128, 5, c, beta), TQ_EINVAL);
  EXPECT(tq_lloyd_max_codebook(128, 3, nullptr, beta), TQ_EINVAL);
}

static void hbm_stream() {
  Buf src(1 << 20), dst(1 << 18), sink(4);
  EXPECT(tq_hbm_stream(src.p, 1 << 20, nullptr, 0, sink.as<uint32_t>(), 16, 0, nullptr), TQ_OK);
  EXPECT(tq_hbm_stream(src.p, 1 << 20, dst.p, 1 << 18, sink.as<uint32_t>(), 64, TQ_STREAM_NONTEMPORAL | TQ_STREAM_LOADS(16),
                       nullptr), TQ_OK);
  EXPECT(tq_hbm_stream(src.p, 1 << 20, dst.p, 1000, sink.as<uint32_t>(), 16, 0, nullptr), TQ_EINVAL);
  EXPECT(tq_hbm_stream(src.p, 1 << 20, nullptr, 0, sink.as<uint32_t>(), 13, 0, nullptr), TQ_EINVAL);
  EXPECT(tq_hbm_stream(src.p, 1 << 20, nullptr, 0, sink.as<uint32_t>(), 16, TQ_STREAM_LOADS(5), nullptr), TQ_EINVAL);
  EXPECT(tq_hbm_stream(nullptr, 1 << 20, nullptr, 0, sink.as<uint32_t>(), 16, 0, nullptr), TQ_EINVAL);
  EXPECT(tq_hbm_stream((char*)src.p + 4, 1 << 19, nullptr, 0, sink.as<uint32_t>(), 16, 0, nullptr), TQ_EINVAL);
}

static void one_shape(int d, int m, int kb, int vb) {
  std::printf("shape d=%d m=%d key_bits=%d value_bits=%d\n", d, m, kb, vb);
  tq_config cfg{d, m, kb, vb};
  std::vector<double> R((size_t)d * d), S((size_t)m * d);
  for (size_t i = 0; i < R.size(); ++i) R[i] = std::sin(0.37 * (double)i + 0.1) / std::sqrt((double)d);
  for (size_t i = 0; i < S.size(); ++i) S[i] = std::cos(0.71 * (double)i);
  tq_ctx* ctx = nullptr;
  EXPECT(tq_create(&cfg, R.data(), S.data(), nullptr), TQ_EINVAL);
  EXPECT(tq_create(&cfg, nullptr, S.data(), &ctx), TQ_EINVAL);
  EXPECT(tq_create(&cfg, R.data(), S.data(), &ctx), TQ_OK);
  if (!ctx) return;
  EXPECT(tq_key_record_bytes(ctx), tq_config_key_record_bytes(&cfg));
  EXPECT(tq_value_record_bytes(ctx) * 128, tq_value_block_bytes(&cfg));

  const int n_seq = 3, G = 8;
  const int64_t cap = 512;
  Buf keys(tq_cache_key_bytes(&cfg, n_seq, cap)), vals(tq_cache_value_bytes(&cfg, n_seq, cap));
  tq_cache_view view{keys.p, vals.p, cap, n_seq};
  Buf x((size_t)n_seq * 300 * d * 4);
  for (size_t i = 0; i < (size_t)n_seq * 300 * d; ++i) x.as<uint16_t>()[i] = half_bits(0.01f * (float)(i % 97) - 0.4f);

  // no codebook yet
  EXPECT(tq_append_key(ctx, &view, x.p, TQ_F16, 0, 1, nullptr), TQ_ENOCODEBOOK);
  for (int b : {kb, vb}) {
    std::vector<double> c(16), beta(16);
    EXPECT(tq_lloyd_max_codebook(d, b, c.data(), beta.data()), TQ_OK);
    EXPECT(tq_codebook_load(ctx, b, c.data(), b ? beta.data() : nullptr), TQ_OK);
    if (b >= 2) {
      std::vector<double> asym(c);
      asym[0] *= 1.5;
      EXPECT(tq_codebook_load(ctx, b, asym.data(), beta.data()), TQ_EINVAL);
      std::vector<double> unsorted(c);
      std::swap(unsorted[0], unsorted[1]);
      EXPECT(tq_codebook_load(ctx, b, unsorted.data(), beta.data()), TQ_EINVAL);
      EXPECT(tq_codebook_load(ctx, b, c.data(), beta.data()), TQ_OK);
    }
  }
  EXPECT(tq_codebook_load(ctx, 5, nullptr, nullptr), TQ_EINVAL);

  // appends: small, bulk, ragged; errors
  int64_t pos = 0;
  for (int64_t n : {1, 16, 17, 200, 0, 5}) {
    EXPECT(tq_append_key(ctx, &view, x.p, TQ_F16, pos, n, nullptr), TQ_OK);
    EXPECT(tq_append_value(ctx, &view, x.p, TQ_F16, pos, n, nullptr), TQ_OK);
    const size_t need = tq_append_workspace_bytes(ctx, n_seq, n);
    Buf ws(need);
    EXPECT(tq_append_key_ws(ctx, &view, x.p, TQ_F32, pos, n, ws.p, need, nullptr), TQ_OK);
    EXPECT(tq_append_value_ws(ctx, &view, x.p, TQ_F32, pos, n, ws.p, need, nullptr), TQ_OK);
    // which appends take the workspace (general-path bulk appends)
    const bool fast = d == 128 && (m == 64 || m == 128);
    const bool k_ws = kb > 0 && n > 16 && !fast, v_ws = n > 16 && d != 128;
    EXPECT(need > 0, k_ws || v_ws);
    EXPECT(tq_append_key_ws(ctx, &view, x.p, TQ_F16, pos, n, ws.p, need ? need - 1 : 0, nullptr),
           k_ws ? TQ_EWORKSPACE : TQ_OK);
    EXPECT(tq_append_value_ws(ctx, &view, x.p, TQ_F16, pos, n, nullptr, need, nullptr), v_ws ? TQ_EINVAL : TQ_OK);
    pos += n;
  }
  EXPECT(tq_append_key(ctx, &view, x.p, TQ_F16, cap - 2, 3, nullptr), TQ_ECAPACITY);
  EXPECT(tq_append_key(ctx, &view, x.p, TQ_F16, -1, 1, nullptr), TQ_ECAPACITY);
  EXPECT(tq_append_key(ctx, &view, x.p, 3, 0, 1, nullptr), TQ_EINVAL);
  EXPECT(tq_append_key(ctx, &view, (char*)x.p + 2, TQ_F16, 0, 1, nullptr), TQ_EINVAL);
  EXPECT(tq_append_value(ctx, &view, nullptr, TQ_F16, 0, 1, nullptr), TQ_EINVAL);
  tq_cache_view bad = view;
  bad.capacity = 100;
  EXPECT(tq_append_key(ctx, &bad, x.p, TQ_F16, 0, 1, nullptr), TQ_EINVAL);
  bad = view;
  bad.key_records = (char*)keys.p + 4;
  EXPECT(tq_append_key(ctx, &bad, x.p, TQ_F16, 0, 1, nullptr), TQ_EINVAL);

  // scores, attend, decode step, no-allocation attend, top-k, reconstruction
  for (int g : {1, G, 16, 40}) {
    const int64_t nt = pos;
    Buf q((size_t)n_seq * g * d * 4), sc((size_t)n_seq * g * nt * 4), out((size_t)n_seq * g * d * 4);
    const size_t need = tq_attend_workspace_bytes(ctx, n_seq, g, nt);
    EXPECT_TRUE(need > 0);
    EXPECT(need, tq_workspace_bytes(&cfg, n_seq, g, nt));
    Buf ws(need);
    EXPECT(tq_attention_scores(ctx, &view, q.p, TQ_F16, g, nt, sc.as<float>(), ws.p, need, nullptr), TQ_OK);
    EXPECT(tq_attention_scores(ctx, &view, q.p, TQ_F16, g, nt, sc.as<float>(), ws.p, 16, nullptr), TQ_EWORKSPACE);
    EXPECT(tq_attend_noalloc(ctx, &view, q.p, TQ_F16, g, nt, 0.f, nullptr, nullptr), TQ_EINVAL);
    EXPECT(tq_attention_scores(ctx, &view, q.p, TQ_F16, g, cap + 1, sc.as<float>(), ws.p, need, nullptr), TQ_EINVAL);
    if (g <= 16) {
      EXPECT(tq_attend(ctx, &view, q.p, TQ_F32, g, nt, 0.f, out.as<float>(), ws.p, need, nullptr), TQ_OK);
      EXPECT(tq_attend_noalloc(ctx, &view, q.p, TQ_F16, g, nt, 0.25f, out.as<float>(), nullptr), TQ_OK);
      const size_t dneed = tq_attend_workspace_bytes(ctx, n_seq, g, nt + 1);
      Buf dws(dneed);
      EXPECT(tq_decode_step(ctx, &view, x.p, x.p, TQ_F16, nt, 1, q.p, g, 0.f, out.as<float>(), dws.p, dneed, nullptr),
             TQ_OK);
      EXPECT(tq_decode_step(ctx, &view, x.p, x.p, TQ_F16, nt, 0, q.p, g, 0.f, out.as<float>(), dws.p, dneed, nullptr),
             TQ_EINVAL);
    } else {
      EXPECT(tq_attend(ctx, &view, q.p, TQ_F16, g, nt, 0.f, out.as<float>(), ws.p, need, nullptr), TQ_EINVAL);
    }
    for (int k : {1, 10, 16}) {
      const size_t tneed = tq_topk_workspace_bytes(&cfg, n_seq, g, nt, k);
      Buf tws(tneed), ts((size_t)n_seq * g * k * 4), ti((size_t)n_seq * g * k * 4);
      EXPECT(tq_topk_scores(ctx, &view, q.p, TQ_F16, g, nt, k, ts.as<float>(), ti.as<int32_t>(), tws.p, tneed, nullptr),
             TQ_OK);
      EXPECT(tq_topk_scores(ctx, &view, q.p, TQ_F16, g, nt, k, ts.as<float>(), ti.as<int32_t>(), tws.p, tneed - 1,
                            nullptr), TQ_EWORKSPACE);
    }
  }
  {
    Buf out((size_t)n_seq * pos * d * 4);
    EXPECT(tq_get_keys(ctx, &view, 0, pos, out.as<float>(), nullptr), TQ_OK);
    EXPECT(tq_get_values(ctx, &view, 3, pos - 3, out.as<float>(), nullptr), TQ_OK);
    EXPECT(tq_get_values(ctx, &view, cap - 3, 4, out.as<float>(), nullptr), TQ_ECAPACITY);
    EXPECT(tq_get_keys(ctx, &view, 0, 0, out.as<float>(), nullptr), TQ_OK);
  }
  EXPECT(tq_destroy(ctx), TQ_OK);
}

int main() {
  size_queries();
  codebooks();
  hbm_stream();
  one_shape(128, 64, 3, 3);
  one_shape(128, 128, 4, 2);
  one_shape(128, 64, 0, 1);
  one_shape(64, 32, 2, 4);
  one_shape(192, 96, 0, 3);
  one_shape(128, 32, 3, 3);
  one_shape(1024, 512, 4, 4);
  EXPECT(tq_destroy(nullptr), TQ_OK);
  std::printf("%d checks, %d failed, %d launches\n", g_checks, g_fail, g_launches);
  if (g_fail) return 1;
  std::printf("ok\n");
  return 0;
}
