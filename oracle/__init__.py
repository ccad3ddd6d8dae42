"""CPU oracle (test infrastructure; see dflash_oracle's header)."""
