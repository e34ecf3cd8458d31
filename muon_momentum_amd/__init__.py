"""MI355X-native Dion3 optimizer-step hot path.

`muon_momentum_amd.dion3` is the ctypes binding of the HIP library (it loads
libdion3.so and raises if it is missing); `muon_momentum_amd.synth` draws the
seeded synthetic inputs.  Importing the package itself loads nothing.
"""
