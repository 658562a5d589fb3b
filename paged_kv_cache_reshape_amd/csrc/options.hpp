// Overrides of the library's own choices, from PAGEDATTN_* environment
// variables.  They are read once, at the first call that needs them, and
// again only when pa_reload_options() is called (tests and tuning runs set
// them; nothing else needs them).
//
//   PAGEDATTN_SCHEDULE=fixed|stream    decode schedule (stream only where built)
//   PAGEDATTN_STREAM_WORKERS=n         stream schedule: worker waves in all
//   PAGEDATTN_DECODE_KERNEL=valu       fixed schedule: vector-ALU kernel only
//   PAGEDATTN_MERGE=separate|inkernel  fixed schedule: where split sequences merge
//   PAGEDATTN_HEADS_PER_WG=1|2|4       fixed schedule: kv heads per workgroup
//   PAGEDATTN_PREFILL_KSPLIT=1|2       prefill: key halves per workgroup
#pragma once

namespace pa {

struct Options {
  int heads_per_wg = 0;    // 0: library choice
  bool valu_only = false;
  int merge = 0;           // 0: library choice, 1: separate kernel, 2: in the launch
  int schedule = 0;        // 0: library choice, 1: fixed partitions, 2: stream
  int stream_workers = 0;  // 0: library choice
  int prefill_ksplit = 0;  // 0: library choice
};

const Options& options();

}  // namespace pa
