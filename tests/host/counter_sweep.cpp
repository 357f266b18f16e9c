// Sweeps the decode entry points over every query length 1..4096 and 1..64 query heads per
// KV head (1, 2 and 8 KV heads, both cache types, page 32 and 64) with the launches stubbed,
// then checks that the launch counters add up: each accepted call counts once in
// decode_launches and once in exactly one of decode_row_tiles / decode_long_windows. Built
// with AddressSanitizer, so a counter index outside its array aborts the run.
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "../../include/fkv.h"

namespace fkv {
extern unsigned long long g_stub_decode_calls;
}

int main() {
  fkv_reset_counters();
  unsigned long long ok[2] = {0, 0}, ok_fused = 0, rejected = 0, expect_tiles[2][7] = {}, expect_long[2] = {0, 0};
  void* dev = reinterpret_cast<void*>(0x100000);
  for (int dt = 0; dt < 2; ++dt) {
    for (int hkv : {1, 2, 8}) {
      for (int bs : {32, 64}) {
        fkv_cache_desc cd{4096, bs, hkv, 128, dt == 0 ? FKV_FP8_E4M3FN : FKV_BF16};
        fkv_cache c;
        if (fkv_init_cache(&cd, dev, dev, &c) != FKV_OK) return 2;
        for (int G = 1; G <= 64; ++G) {
          for (int q_len = 1; q_len <= 4096; ++q_len) {
            fkv_decode_desc d;
            std::memset(&d, 0, sizeof(d));
            d.num_seqs = 1;
            d.q_len = q_len;
            d.num_q_heads = G * hkv;
            d.max_blocks_per_seq = 8192 / bs;
            d.max_seq_len = 8192;
            d.window_left = (q_len % 3 == 0) ? 511 : -1;
            d.softmax_scale = 0.088388f;
            d.out_dtype = FKV_OUT_F32;
            const int nt = (G * q_len + 15) / 16;
            const bool decode_shape = nt <= 7 && q_len <= 16;
            int rc = fkv_decode_attn(&c, &d, (const uint16_t*)dev, (const int32_t*)dev, (const int32_t*)dev,
                                     (const float*)dev, (const float*)dev, dev, dev, (size_t)-1, nullptr);
            if (rc == FKV_OK) {
              ++ok[dt];
              if (decode_shape) ++expect_tiles[dt][nt - 1]; else ++expect_long[dt];
            } else {
              ++rejected;
            }
            if (q_len <= 16) {
              rc = fkv_insert_decode(&c, &d, (const uint16_t*)dev, (const uint16_t*)dev, (const uint16_t*)dev,
                                     (const int32_t*)dev, (const int32_t*)dev, (const float*)dev, (const float*)dev,
                                     dev, dev, (size_t)-1, nullptr);
              if (rc == FKV_OK) {
                ++ok[dt];
                ++ok_fused;
                if (decode_shape) ++expect_tiles[dt][nt - 1]; else ++expect_long[dt];
              } else {
                ++rejected;
              }
            }
          }
        }
      }
    }
  }
  fkv_counters cnt;
  if (fkv_get_counters(&cnt) != FKV_OK) return 3;
  int bad = 0;
  for (int i = 0; i < 2; ++i) {
    unsigned long long tiles = 0;
    for (int j = 0; j < 7; ++j) {
      tiles += cnt.decode_row_tiles[i][j];
      if (cnt.decode_row_tiles[i][j] != expect_tiles[i][j]) ++bad;
    }
    if (cnt.decode_launches[i] != ok[i] || tiles + cnt.decode_long_windows[i] != ok[i]) ++bad;
    if (cnt.decode_long_windows[i] != expect_long[i]) ++bad;
  }
  if (cnt.insert_decode_launches != ok_fused || cnt.rejected_calls != rejected) ++bad;
  if (fkv::g_stub_decode_calls != ok[0] + ok[1]) ++bad;
  std::printf("accepted fp8 %llu bf16 %llu (fused %llu), rejected %llu, long windows fp8 %llu, mismatches %d\n",
              ok[0], ok[1], ok_fused, rejected, (unsigned long long)cnt.decode_long_windows[0], bad);
  return bad ? 1 : 0;
}
