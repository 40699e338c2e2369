"""CPU reference for NVFP4 paged attention.  Test infrastructure only: the
library never imports it; tests, the smoke check and the benchmark's CPU
baseline do."""
