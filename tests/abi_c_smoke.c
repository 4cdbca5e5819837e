/* Plain C99 consumer of include/vocoder.h: compiled with -std=c99 -Wall
 * -Werror -pedantic and run without a GPU.  Calls every entry point through
 * an early-return (validation) path; never touches a device. */
#include <stdio.h>
#include <string.h>
#include "vocoder.h"

#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) {                                                \
      fprintf(stderr, "FAIL line %d: %s\n", __LINE__, #cond);     \
      return 1;                                                   \
    }                                                             \
  } while (0)

int main(void) {
  voc_config cfg;
  voc_ctx *ctx = (voc_ctx *)0;
  voc_profile_stat st;
  int64_t a, b, c;
  double peak = 0.0;
  float dummy[4];
  voc_config_default(&cfg);
  EXPECT(cfg.abi_version == VOC_ABI_VERSION);
  EXPECT(voc_config_validate(&cfg) == VOC_OK);
  EXPECT(voc_config_hop(&cfg) == 512);
  EXPECT(voc_config_halo(&cfg) == 10);
  /* the last ConvTranspose1d reads 256 frames per latent frame */
  EXPECT(voc_config_max_frames(&cfg) > 200000 && voc_config_max_frames(&cfg) < 270000);
  EXPECT(voc_config_max_frames(NULL) == VOC_INVALID_PARAMS);
  EXPECT(cfg.in_proj == 0);
  cfg.in_proj = 1024;
  EXPECT(voc_config_validate(&cfg) == VOC_OK);
  cfg.in_proj = 24;
  EXPECT(voc_config_validate(&cfg) == VOC_INVALID_PARAMS);
  cfg.in_proj = 0;
  EXPECT(cfg.causal == 0);
  cfg.causal = 1;
  EXPECT(voc_config_validate(&cfg) == VOC_OK);
  EXPECT(voc_config_halo(&cfg) > 10);
  cfg.causal = 2;
  EXPECT(voc_config_validate(&cfg) == VOC_INVALID_PARAMS);
  cfg.causal = 0;
  EXPECT(voc_config_validate(NULL) == VOC_INVALID_PARAMS);
  cfg.abi_version = VOC_ABI_VERSION + 1;
  EXPECT(voc_config_validate(&cfg) == VOC_INVALID_PARAMS);
  EXPECT(vocoder_create(&cfg, 0, &ctx) == VOC_INVALID_PARAMS);
  EXPECT(ctx == (voc_ctx *)0);
  EXPECT(strlen(vocoder_last_error(NULL)) > 0);
  EXPECT(vocoder_create(NULL, 0, &ctx) == VOC_INVALID_PARAMS);
  EXPECT(vocoder_create(&cfg, 0, NULL) == VOC_INVALID_PARAMS);
  EXPECT(vocoder_load_weights(NULL, NULL, 0) == VOC_INVALID_PARAMS);
  EXPECT(vocoder_output_length(NULL, 5) == -1);
  EXPECT(vocoder_decode(NULL, dummy, 1, 1, dummy, NULL) == VOC_INVALID_PARAMS);
  EXPECT(vocoder_decode_windows(NULL, dummy, 3, 2, 689, 683, 86, 258, dummy, NULL) == VOC_INVALID_PARAMS);
  EXPECT(vocoder_windows_output_length(NULL, 3, 689, 683, 86, 258) == -1);
  EXPECT(vocoder_stream_reset(NULL, 4) == VOC_INVALID_PARAMS);
  EXPECT(vocoder_encode(NULL, dummy, 1, 1, dummy, NULL) == VOC_INVALID_PARAMS);
  EXPECT(vocoder_set_cancel(NULL, (voc_cancel_fn)0, NULL, 1) == VOC_INVALID_PARAMS);
  EXPECT(VOC_CANCELLED == -6);
  voc_config_default(&cfg);
  cfg.enc_width[0] = 64; cfg.enc_width[1] = 128; cfg.enc_width[2] = 256; cfg.enc_width[3] = 512;
  cfg.enc_width[4] = 1024;
  EXPECT(voc_config_validate(&cfg) == VOC_OK);
  cfg.enc_width[2] = 24;
  EXPECT(voc_config_validate(&cfg) == VOC_INVALID_PARAMS);
  memset(cfg.enc_width, 0, sizeof(cfg.enc_width));
  EXPECT(vocoder_stream_decode(NULL, dummy, 1, dummy, NULL) == VOC_INVALID_PARAMS);
  EXPECT(vocoder_profile_enable(NULL, 1) == VOC_INVALID_PARAMS);
  EXPECT(vocoder_profile_reset(NULL) == VOC_INVALID_PARAMS);
  EXPECT(vocoder_profile_read(NULL, 0, &st) == VOC_INVALID_PARAMS);
  EXPECT(voc_dbg_stage_count(NULL) == VOC_INVALID_PARAMS);
  EXPECT(voc_dbg_stage_shape(NULL, 0, 1, &a, &b, &c) == VOC_INVALID_PARAMS);
  EXPECT(voc_dbg_run_stage(NULL, 0, dummy, 1, 1, dummy, NULL) == VOC_INVALID_PARAMS);
  EXPECT(voc_dbg_copy(NULL, dummy, 16, NULL) == VOC_INVALID_PARAMS);
  EXPECT(voc_dbg_peak(0, 16, NULL, NULL) == VOC_INVALID_PARAMS);
  EXPECT(voc_dbg_peak(5, 16, &peak, NULL) == VOC_INVALID_PARAMS);
  EXPECT(voc_dbg_peak(0, 10, &peak, NULL) == VOC_INVALID_PARAMS);
  vocoder_destroy(NULL);
  puts("abi ok");
  return 0;
}
